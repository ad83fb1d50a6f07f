"""Attention visibility over X~ = [R, X] (meta tokens first), and the ring slot
of the decode KV cache.

Sources:
* Meta tokens are prepended and interact with every later token, also in
  sliding-window layers — Hymba blog, "Hymba简介"; "数学表示" §1 defines
  X~ = [R, X].
* Sliding-window layers attend a local window; the first, middle and last
  blocks are global — Hymba blog, "Hymba 的整体架构".

Readings (the pages give no index arithmetic):
* Rows i and columns j index the concatenated X~ (meta rows 0..M-1).
* Causal everywhere: j <= i (meta rows see only earlier meta rows).
* The window holds the W most recent rows, the query itself included:
  i - j < W.  W <= 0 means global (no window).
* Meta keys are always visible to later rows; meta and window visibility are a
  union (no key counted twice).
"""
from __future__ import annotations

import numpy as np


def visible(i: int, j: int, n_meta: int, window: int) -> bool:
    """Scalar predicate: may query row i attend key row j?"""
    if j > i:
        return False
    if j < n_meta or window <= 0:
        return True
    return i - j < window


def mask_rows(rows, T: int, n_meta: int, window: int) -> np.ndarray:
    """Boolean [len(rows), T] visibility for the given query rows."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(T, dtype=np.int64)[None, :]
    m = j <= i
    if window > 0:
        m = m & ((j < n_meta) | (i - j < window))
    return m


def mask(T: int, n_meta: int, window: int) -> np.ndarray:
    """Boolean [T, T] visibility matrix."""
    return mask_rows(np.arange(T), T, n_meta, window)


def visible_count(T: int, n_meta: int, window: int) -> np.ndarray:
    """Number of visible keys per query row (row sums of the mask)."""
    return mask(T, n_meta, window).sum(axis=1)


def tile_kinds(T: int, n_meta: int, window: int, bm: int, bn: int) -> np.ndarray:
    """Classify each (query tile, key tile) block of the mask.

    Returns int32 [ceil(T/bm), ceil(T/bn)]: 0 = no visible pair (skipped),
    1 = some but not all pairs visible (needs the element mask),
    2 = every pair visible.  Ragged last tiles count only their real rows and
    columns.  Derived by counting mask entries, nothing else.
    """
    m = mask(T, n_meta, window)
    nq, nk = -(-T // bm), -(-T // bn)
    out = np.zeros((nq, nk), dtype=np.int32)
    for a in range(nq):
        for b in range(nk):
            blk = m[a * bm:(a + 1) * bm, b * bn:(b + 1) * bn]
            c = int(blk.sum())
            out[a, b] = 0 if c == 0 else (2 if c == blk.size else 1)
    return out


def cache_slot(n_prev: int, n_meta: int, window: int) -> int:
    """Cache row that receives the token at position n_meta + n_prev.

    Reading: slots 0..M-1 hold the meta tokens; a sliding-window layer keeps a
    ring of W slots after them (token s lives in slot M + s mod W); a global
    layer appends (slot M + s).
    """
    if n_prev < 0:
        raise ValueError("n_prev must be >= 0")
    return n_meta + (n_prev % window if window > 0 else n_prev)
