"""Whole Hymba blocks around the mixer core, and their stack (prefill).

Sources:
* Hymba blog (juejin.cn, "NVIDIA提出Hymba网络"), "Hymba 的整体架构": a block is a
  normalisation layer, the hybrid-head module, a second normalisation layer and
  a feed-forward network; the first, middle and last blocks attend to all
  tokens, the others through a sliding window, and adjacent sliding-window
  blocks share one KV cache.
* Same page, "数学表示" §2 (X~ times W_in_proj gives Q, K, V, the SSM input and
  the gate), §4 (Eq. (2): Delta, B, C indexed by time) and §5 (W_out_proj maps
  the fused heads back to the model width).
* Hymba-1.5B-Base model card, "模型架构": width 1600, MLP intermediate width
  5504, 32 layers.

Readings (the pages leave these open):
* Residual form (pre-norm): each half of the block adds its result to the
  running hidden state,
      h1 = h + W_out mixer(norm1(h)),   h2 = h1 + FFN(norm2(h1)).
* The two normalisation layers are RMS norms over the model width with a
  learned weight, the same eps as the branch norms.
* FFN: two matrices with SiLU between them, FFN(u) = W_down SiLU(W_up u).
* Delta, B and C: Eq. (2) indexes them by time, so they depend on the input.
  They are taken from the SSM input x (the W_SSM part of the in-projection)
  by one more projection W_dbc [Di + 2 Ns, Di]:
      Delta = softplus(x W_dt^T + dt_bias),  B = x W_B^T,  C = x W_C^T,
  with W_dbc's rows in the order W_dt, W_B, W_C.  softplus keeps the step
  sizes non-negative, as the mixer core requires.
* A block that reuses its neighbour's KV cache has no W_K, W_V: its
  in-projection gives Q, x and z only, and its attention reads the producer's
  K and V (which the producer made from its own input).
"""
from __future__ import annotations

import numpy as np

from .linear import linear, split_columns
from .mixer import mixer_prefill


def rms_norm(x, w, eps: float = 1e-6):
    """x [..., width] / sqrt(mean(x^2) + eps) * w [width], float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), computed without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def ffn(u, w_up, w_down):
    """W_down SiLU(W_up u): u [..., d], w_up [F, d], w_down [d, F]."""
    return linear(silu(linear(u, w_up)), w_down)


def block_prefill(hidden, p: dict, Hq: int, Hkv: int, Dh: int, n_meta: int, window: int,
                  kv=None, rope_base: float = 10000.0, eps: float = 1e-6, pos0: int = 0) -> dict:
    """One block over X~'s hidden states ``hidden`` [B, T, d].

    ``p`` holds ln1, ln2 [d]; w_in [Hq Dh + 2 Hkv Dh + 2 Di, d] (producer) or
    [Hq Dh + 2 Di, d] (``kv`` given: the block reuses that K, V); w_dbc
    [Di + 2 Ns, Di]; dt_bias [Di]; A, D, conv_w, conv_b, beta_a, beta_s as for
    the mixer; w_out [d, Di]; w_up [F, d]; w_down [d, F].
    ``kv`` = (k, v) [B, T, Hkv, Dh] of the producer block, or None.
    Returns float64 ``hidden`` (h2), ``mid`` (h1), ``mixer_out`` and the
    block's ``k``, ``v`` (its own, or the reused ones)."""
    h = np.asarray(hidden, dtype=np.float64)
    B, T, _ = h.shape
    Di = np.asarray(p["A"]).shape[0]
    Ns = np.asarray(p["A"]).shape[1]
    u = rms_norm(h, p["ln1"], eps)
    proj = linear(u, p["w_in"])
    if kv is None:
        q, k, v, x, z = split_columns(proj, [Hq * Dh, Hkv * Dh, Hkv * Dh, Di, Di])
        k = k.reshape(B, T, Hkv, Dh)
        v = v.reshape(B, T, Hkv, Dh)
    else:
        q, x, z = split_columns(proj, [Hq * Dh, Di, Di])
        k, v = (np.asarray(t, dtype=np.float64) for t in kv)
    dt, Bm, Cm = split_columns(linear(x, p["w_dbc"]), [Di, Ns, Ns])
    inp = {"q": q.reshape(B, T, Hq, Dh), "k": k, "v": v, "x": x,
           "delta": softplus(dt + np.asarray(p["dt_bias"], np.float64)), "Bm": Bm, "Cm": Cm,
           "z": z}
    for key in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s"):
        inp[key] = np.asarray(p[key], dtype=np.float64)
    mo = mixer_prefill(inp, n_meta, window, rope_base, eps, pos0)["out"]
    h1 = h + linear(mo, p["w_out"])
    h2 = h1 + ffn(rms_norm(h1, p["ln2"], eps), p["w_up"], p["w_down"])
    return {"hidden": h2, "mid": h1, "mixer_out": mo, "k": k, "v": v}


def stack_prefill(hidden, layers, roles, Hq: int, Hkv: int, Dh: int, n_meta: int,
                  rope_base: float = 10000.0, eps: float = 1e-6, pos0: int = 0) -> dict:
    """Blocks chained: ``layers[l]`` holds block l's weights, ``roles[l]`` =
    (window, kv_source_layer); a block whose source is an earlier layer reuses
    that layer's K, V.  Returns the final hidden states and each block's
    output (``per_layer``), float64."""
    h = np.asarray(hidden, dtype=np.float64)
    kvs, outs = {}, []
    for l, (p, (window, src)) in enumerate(zip(layers, roles)):
        r = block_prefill(h, p, Hq, Hkv, Dh, n_meta, window,
                          None if src == l else kvs[src], rope_base, eps, pos0)
        kvs[l] = (r["k"], r["v"])
        h = r["hidden"]
        outs.append(h)
    return {"hidden": h, "per_layer": outs}
