"""Normalise each branch, rescale by a learnable vector, and average.

Sources: the SSM output is larger in magnitude than the attention output, so
both are normalised before fusion and then averaged — Hymba blog,
"深入理解混合头模块"; the fusion beta_1 * norm(Y_attn) + beta_2 * norm(Y_ssm)
with learnable vectors beta — "数学表示" §5; "outputs of the blocks are
averaged", with a norm after head concatenation — Telegram post
"Mamba, Jamba, Ху...Hymba!".

Readings:
* §5 prints a sum, the prose says average: out = 0.5 * (sum).
* norm is an RMS norm per token over the whole branch width (all heads
  concatenated), no mean removal, no bias; beta is its weight.
* eps = 1e-6 inside the square root.
"""
from __future__ import annotations

import numpy as np


def rms_normalize(y, eps: float = 1e-6):
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)


def branch_norm_mean(ya, ys, beta_a, beta_s, eps: float = 1e-6):
    """ya, ys [..., width]; beta_a, beta_s [width] -> [..., width] float64."""
    ba = np.asarray(beta_a, dtype=np.float64)
    bs = np.asarray(beta_s, dtype=np.float64)
    return 0.5 * (ba * rms_normalize(ya, eps) + bs * rms_normalize(ys, eps))
