"""One decode token through one layer of an adjacent pair sharing a KV cache.

Sources: generation with the KV cache enabled — Hymba-1.5B-Base model card,
"模型使用" step 2; adjacent sliding-window blocks share one KV cache instead of
keeping their own — Hymba blog, "Hymba 的整体架构"; meta tokens are fixed and
at the start of every sequence — Hymba blog, "深入理解元 Tokens"; one
sequence length for the whole batch (batched generation with padded meta
tokens under a sliding window is not supported) — Chinese news article,
"不過，需要小心".

Readings:
* Cache rows: 0..M-1 meta tokens, then a ring of W slots (token s in slot
  M + s mod W; global layers append).  K is stored already rotated.
* The new token sits at position p = M + n_prev.  The producer layer rotates
  k_new at p and writes k_new/v_new into its slot before attending, so the
  token sees itself; the consumer layer writes nothing and reads the same cache
  with its own q.
* Visible slots: the meta rows and the ring slots of the last min(n_prev+1, W)
  tokens.  Order does not matter (positions live in the rotated K).
* The conv and SSM states advance by one token; then norm-and-average.
* Ragged batches (``mixer_step_ragged``): the news article's limitation is a
  property of that implementation, not of the method; every sequence is an
  independent instance of the step above at its own n_prev.
"""
from __future__ import annotations

import numpy as np

from .conv import conv_step
from .mask import cache_slot
from .norm import branch_norm_mean
from .rope import rope, rope_at
from .scan import scan_step


def valid_slots(n_prev: int, n_meta: int, window: int) -> np.ndarray:
    """Cache rows a token at position n_meta + n_prev may attend (after its write)."""
    if window > 0:
        cnt = min(n_prev + 1, window)
        ring = [n_meta + ((n_prev - s) % window) for s in range(cnt)]
    else:
        ring = [n_meta + s for s in range(n_prev + 1)]
    return np.array(list(range(n_meta)) + sorted(ring), dtype=np.int64)


def build_cache(k, v, n_meta: int, n_tokens: int, window: int, cache_slots: int,
                rope_base: float = 10000.0, fill=None):
    """Cache after prefill of the first n_meta + n_tokens rows of k, v.

    k, v [B, T', Hkv, Dh] (pre-RoPE, T' >= n_meta + n_tokens).  Returns float64
    (k_cache, v_cache) [B, n_meta + cache_slots, Hkv, Dh]; rows never written
    hold ``fill`` (default NaN, so reading one shows up).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, _, Hkv, Dh = k.shape
    S = n_meta + cache_slots
    kc = np.full((B, S, Hkv, Dh), np.nan if fill is None else fill)
    vc = kc.copy()
    L = n_meta + n_tokens
    kr = rope(k[:, :L], np.arange(L), rope_base)
    kc[:, :n_meta] = kr[:, :n_meta]
    vc[:, :n_meta] = v[:, :n_meta]
    first = max(0, n_tokens - window) if window > 0 else 0
    for s in range(first, n_tokens):
        slot = cache_slot(s, n_meta, window)
        if slot >= S:
            raise ValueError("cache too small")
        kc[:, slot] = kr[:, n_meta + s]
        vc[:, slot] = v[:, n_meta + s]
    return kc, vc


def mixer_step(layer: dict, k_cache, v_cache, n_prev: int, n_meta: int,
               window: int, producer: bool, rope_base: float = 10000.0,
               eps: float = 1e-6, scale: float = 0.0) -> dict:
    """``layer`` holds q [B, Hq, Dh], (k_new, v_new [B, Hkv, Dh] if producer),
    x, delta, z [B, Di], Bm, Cm [B, N], conv_state [B, Di, K-1],
    ssm_state [B, Di, N], A, D, conv_w, conv_b, beta_a, beta_s.

    Returns float64 out, ya, ys [B, Di], the advanced states and the cache
    (a modified copy when ``producer``)."""
    q = np.asarray(layer["q"], dtype=np.float64)
    B, Hq, Dh = q.shape
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    Hkv = kc.shape[2]
    grp = Hq // Hkv
    p = n_meta + n_prev
    if producer:
        slot = cache_slot(n_prev, n_meta, window)
        if slot >= kc.shape[1]:
            raise ValueError("cache too small")
        kc[:, slot] = rope_at(layer["k_new"], p, rope_base)
        vc[:, slot] = np.asarray(layer["v_new"], dtype=np.float64)
    rows = valid_slots(n_prev, n_meta, window)
    if rows.max() >= kc.shape[1]:
        raise ValueError("cache too small")
    s = 1.0 / np.sqrt(Dh) if scale <= 0 else float(scale)
    qr = rope_at(q, p, rope_base)
    o = np.empty((B, Hq, Dh))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            sc = kc[b, rows, g, :] @ qr[b, h] * s
            w = np.exp(sc - sc.max())
            o[b, h] = (w / w.sum()) @ vc[b, rows, g, :]
    ya = o.reshape(B, Hq * Dh)
    xc, conv_state = conv_step(layer["x"], layer["conv_w"], layer["conv_b"],
                               layer["conv_state"], True)
    ys, h = scan_step(xc, layer["delta"], layer["A"], layer["Bm"], layer["Cm"],
                      layer["D"], layer["z"], layer["ssm_state"])
    out = branch_norm_mean(ya, ys, layer["beta_a"], layer["beta_s"], eps)
    return {"out": out, "ya": ya, "ys": ys, "conv_state": conv_state,
            "ssm_state": h, "k_cache": kc, "v_cache": vc}


_SEQ_KEYS = ("q", "k_new", "v_new", "x", "delta", "z", "Bm", "Cm", "conv_state", "ssm_state")


def mixer_step_ragged(layer: dict, k_cache, v_cache, n_prev_seq, n_meta: int,
                      window: int, producer: bool, rope_base: float = 10000.0,
                      eps: float = 1e-6, scale: float = 0.0) -> dict:
    """``mixer_step`` with one n_prev per sequence: sequence b is the step of
    that sequence alone at n_prev_seq[b].  Same arguments and results."""
    B = np.asarray(layer["q"]).shape[0]
    outs = []
    for b in range(B):
        lb = {k: (np.asarray(v)[b:b + 1] if k in _SEQ_KEYS and v is not None else v)
              for k, v in layer.items()}
        outs.append(mixer_step(lb, np.asarray(k_cache)[b:b + 1], np.asarray(v_cache)[b:b + 1],
                               int(n_prev_seq[b]), n_meta, window, producer, rope_base, eps,
                               scale))
    return {k: np.concatenate([o[k] for o in outs], axis=0) for k in outs[0]}
