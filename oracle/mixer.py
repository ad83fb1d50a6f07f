"""One hybrid-head mixer layer over already-projected inputs (prefill).

Source: Hymba blog, "数学表示" §6 (summary of the module): X~ -> projections
-> attention heads and SSM heads in parallel -> normalise, rescale, average.
The projections W_in_proj / W_out_proj (§2, §5) are outside this core: the
inputs here are Q, K, V and the SSM inputs x, Delta, B, C, z.

Composition: attention (Eq. (1)) reshaped to [B, T, Hq*Dh]; causal conv then
selective scan (Eq. (2)) starting from zero state; branch norm-and-average.

Cached meta tokens: the meta tokens are learned constants placed in front of
every sequence (Hymba blog, "Hymba 的整体架构": learnable meta tokens prepended
to the input), so within one layer their projected rows, hence their K and V
and the SSM-branch states after them, are the same for every prompt.
``meta_cache`` takes those constants from the meta rows once;
``mixer_prefill_cached_meta`` then computes only the real-token rows: the
attention keys are the cached meta rows followed by the tokens (visibility and
positions as over X~ = [meta; tokens]) and the SSM branch starts from the
cached states.  Reading: the pages do not describe this precomputation; it
follows from the meta tokens being input-independent.
"""
from __future__ import annotations

import numpy as np

from .attention import attention
from .conv import causal_conv1d
from .norm import branch_norm_mean
from .scan import selective_scan


def mixer_prefill(inp: dict, n_meta: int, window: int, rope_base: float = 10000.0,
                  eps: float = 1e-6, pos0: int = 0, scale: float = 0.0) -> dict:
    """``inp`` holds q, k, v, x, delta, Bm, Cm, z, A, D, conv_w, conv_b, beta_a,
    beta_s as produced by the workload generator.  Returns float64 ya, ys, out
    [B, T, Di] and the final conv and SSM states."""
    q = np.asarray(inp["q"])
    B, T, Hq, Dh = q.shape
    ya = attention(q, inp["k"], inp["v"], n_meta, window, rope_base, pos0,
                   scale).reshape(B, T, Hq * Dh)
    xc, conv_state = causal_conv1d(inp["x"], inp["conv_w"], inp["conv_b"], None, True)
    ys, h = selective_scan(xc, inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                           inp["D"], inp["z"], None)
    out = branch_norm_mean(ya, ys, inp["beta_a"], inp["beta_s"], eps)
    return {"ya": ya, "ys": ys, "out": out, "ssm_state": h, "conv_state": conv_state}


def meta_cache(meta: dict) -> dict:
    """``meta`` holds the M meta rows of one sequence (k, v [M, Hkv, Dh]; x,
    delta, Bm, Cm [M, ...]; conv_w, conv_b, A).  Returns the cached constants:
    k, v (pre-RoPE, as given) and the conv and SSM states after the M rows
    (conv_state [Di, K-1], ssm_state [Di, N]), float64."""
    x = np.asarray(meta["x"], dtype=np.float64)[None]
    xc, conv_state = causal_conv1d(x, meta["conv_w"], meta["conv_b"], None, True)
    _, h = selective_scan(xc, np.asarray(meta["delta"])[None], meta["A"],
                          np.asarray(meta["Bm"])[None], np.asarray(meta["Cm"])[None],
                          None, None, None)
    return {"k": np.asarray(meta["k"], dtype=np.float64),
            "v": np.asarray(meta["v"], dtype=np.float64),
            "conv_state": conv_state[0], "ssm_state": h[0]}


def mixer_prefill_cached_meta(inp: dict, cache: dict, n_meta: int, window: int,
                              rope_base: float = 10000.0, eps: float = 1e-6, pos0: int = 0,
                              scale: float = 0.0) -> dict:
    """``inp`` holds the real-token rows only (q, k, v, x, ... [B, N, ...]);
    ``cache`` is ``meta_cache`` of the layer's meta rows (n_meta of them).
    Token i sits at X~ row n_meta + i (position pos0 + n_meta + i).  Returns
    float64 ya, ys, out [B, N, Di] and the final conv and SSM states."""
    q = np.asarray(inp["q"], dtype=np.float64)
    B, N, Hq, Dh = q.shape
    M = n_meta
    mk = np.broadcast_to(cache["k"], (B,) + cache["k"].shape)
    mv = np.broadcast_to(cache["v"], (B,) + cache["v"].shape)
    kk = np.concatenate([mk, np.asarray(inp["k"], dtype=np.float64)], axis=1)
    vv = np.concatenate([mv, np.asarray(inp["v"], dtype=np.float64)], axis=1)
    qq = np.concatenate([np.zeros((B, M, Hq, Dh)), q], axis=1)   # meta queries unused
    ya = attention(qq, kk, vv, M, window, rope_base, pos0, scale,
                   rows=M + np.arange(N)).reshape(B, N, Hq * Dh)
    cs = np.broadcast_to(cache["conv_state"], (B,) + cache["conv_state"].shape)
    h0 = np.broadcast_to(cache["ssm_state"], (B,) + cache["ssm_state"].shape)
    xc, conv_state = causal_conv1d(inp["x"], inp["conv_w"], inp["conv_b"], cs, True)
    ys, h = selective_scan(xc, inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                           inp["D"], inp["z"], h0)
    out = branch_norm_mean(ya, ys, inp["beta_a"], inp["beta_s"], eps)
    return {"ya": ya, "ys": ys, "out": out, "ssm_state": h, "conv_state": conv_state}
