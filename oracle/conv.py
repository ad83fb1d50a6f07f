"""Causal depthwise conv1d in front of the selective scan.

The pages do not describe this step (the SSM input is W_SSM X~, Hymba blog
"数学表示" §2); it is the short convolution of a Mamba head, width K = 4.

Readings:
* Cross-correlation over time per channel: u[t, c] = b[c] + sum_k w[c, k] *
  x[t - K + 1 + k, c], so w[c, K-1] multiplies the current token.
* Inputs before t = 0 come from ``state_in`` (the previous K-1 inputs, oldest
  first) or are zero.
* Output activation SiLU(u) = u * sigmoid(u) when ``apply_silu``.
* ``state_out`` is the last K-1 inputs (oldest first): what a following call,
  or a decode step, needs.
"""
from __future__ import annotations

import numpy as np


def causal_conv1d(x, w, bias=None, state_in=None, apply_silu: bool = True):
    """x [B, T, Di], w [Di, K], bias [Di] | None, state_in [B, Di, K-1] | None.

    Returns (y [B, T, Di], state_out [B, Di, K-1]), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, Di = x.shape
    K = w.shape[1]
    if state_in is None:
        prev = np.zeros((B, K - 1, Di))
    else:
        prev = np.asarray(state_in, dtype=np.float64).transpose(0, 2, 1)
    xp = np.concatenate([prev, x], axis=1)            # [B, K-1+T, Di]
    u = np.zeros((B, T, Di))
    if bias is not None:
        u += np.asarray(bias, dtype=np.float64)
    for kk in range(K):
        u += w[:, kk] * xp[:, kk:kk + T, :]
    y = u / (1.0 + np.exp(-u)) if apply_silu else u
    state_out = xp[:, T:T + K - 1, :].transpose(0, 2, 1).copy()
    return y, state_out


def conv_step(x, w, bias, state, apply_silu: bool = True):
    """One token: x [B, Di], state [B, Di, K-1] -> (y [B, Di], new state)."""
    y, st = causal_conv1d(np.asarray(x, dtype=np.float64)[:, None, :], w, bias,
                          state, apply_silu)
    return y[:, 0, :], st
