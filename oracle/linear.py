"""The projections around the mixer.

Source: Hymba blog, "数学表示" §2: X~ times W_in_proj gives Q, K, V, the SSM
input and the gate G; §5: W_out_proj maps the fused output back.  The weight
is in nn.Linear layout ([N, K]): y = x W^T.

Readings:
* The in-projection's output columns are taken in the order Q, K, V, SSM input
  x, gate z, each a consecutive block of columns (the pages name the pieces,
  not their order or packing).  The SSM's Delta, B and C are not part of this
  projection (the pages derive them from the SSM input; they stay inputs of
  the mixer here).
"""
from __future__ import annotations

import numpy as np


def linear(x, w):
    """x [..., K], w [N, K] -> x w^T [..., N], float64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def split_columns(y, seg_cols):
    """Consecutive column blocks of widths seg_cols (summing to y's last dim)."""
    y = np.asarray(y)
    edges = np.cumsum([0] + list(seg_cols))
    if edges[-1] != y.shape[-1]:
        raise ValueError("segment widths must sum to the number of columns")
    return [y[..., a:b] for a, b in zip(edges[:-1], edges[1:])]
