"""One hybrid-head mixer layer over already-projected inputs (prefill).

Source: Hymba blog, "数学表示" §6 (summary of the module): X~ -> projections
-> attention heads and SSM heads in parallel -> normalise, rescale, average.
The projections W_in_proj / W_out_proj (§2, §5) are outside this core: the
inputs here are Q, K, V and the SSM inputs x, Delta, B, C, z.

Composition: attention (Eq. (1)) reshaped to [B, T, Hq*Dh]; causal conv then
selective scan (Eq. (2)) starting from zero state; branch norm-and-average.
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
