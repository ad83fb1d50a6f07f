"""Rotary position embedding on queries and keys.

Source: RoPE is named in the Hymba-1.5B-Base model card, "模型架构" (model
architecture); the pages give no formula.

Reading: the rotate-half form. For head dim Dh and d < Dh/2 the pair
(x[d], x[d + Dh/2]) is rotated by the angle pos * base**(-2d/Dh), with base
10000. Row i of X~ has position pos0 + i, so meta tokens take positions
0..M-1 (they are rows of X~, Hymba blog "数学表示" §1). Angles are float64.
"""
from __future__ import annotations

import numpy as np


def rope_angles(pos, Dh: int, base: float) -> np.ndarray:
    """float64 [len(pos), Dh/2] rotation angles."""
    half = Dh // 2
    theta = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / Dh)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate x[B, T, H, Dh] at positions pos[T]."""
    x = np.asarray(x, dtype=np.float64)
    Dh = x.shape[-1]
    half = Dh // 2
    ang = rope_angles(pos, Dh, base)[None, :, None, :]   # [1, T, 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_at(x: np.ndarray, p: int, base: float) -> np.ndarray:
    """Rotate x[B, H, Dh] (one token per sequence) at the single position p."""
    x = np.asarray(x, dtype=np.float64)
    return rope(x[:, None], [p], base)[:, 0]
