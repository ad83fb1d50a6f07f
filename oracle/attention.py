"""Attention heads over X~ with GQA, RoPE, a sliding window and meta tokens.

Source: Hymba blog, "数学表示" §3, Eq. (1): Y_attn = softmax(Q K^T) V, with Q,
K, V the projections of X~ (§2).  GQA — Hymba-1.5B-Base model card,
"模型架构"; KV shared between heads of a layer — model card, "模型概述".

Readings:
* Eq. (1) prints no scale; the standard 1/sqrt(Dh) is used (scale <= 0), and
  an explicit scale may be passed.
* GQA map: query head h reads KV head floor(h / (Hq / Hkv)) (contiguous groups).
* Masked entries take no probability; visibility as in ``oracle.mask``.

This is the plain definition: scores, mask, softmax over the visible keys of a
row, weighted sum of V.  Query rows are processed in blocks only to bound
memory.
"""
from __future__ import annotations

import numpy as np

from .mask import mask_rows
from .rope import rope


def attention(q, k, v, n_meta: int, window: int, rope_base: float = 10000.0,
              pos0: int = 0, scale: float = 0.0, rows=None, block: int = 512):
    """q [B, T, Hq, Dh], k/v [B, T, Hkv, Dh] (pre-RoPE) -> O [B, R, Hq, Dh].

    ``rows`` selects query rows (default: all T); the result holds them in the
    given order.  float64 throughout.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, Dh = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    s = 1.0 / np.sqrt(Dh) if scale <= 0 else float(scale)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    kr = rope(k, pos0 + np.arange(T), rope_base)
    out = np.empty((B, len(rows), Hq, Dh), dtype=np.float64)
    for start in range(0, len(rows), block):
        r = rows[start:start + block]
        m = mask_rows(r, T, n_meta, window)
        qr = rope(q[:, r], pos0 + r, rope_base)
        for b in range(B):
            for h in range(Hq):
                g = h // grp
                sc = (qr[b, :, h, :] @ kr[b, :, g, :].T) * s
                sc = np.where(m, sc, -np.inf)
                sc = sc - sc.max(axis=1, keepdims=True)
                p = np.exp(sc)
                p /= p.sum(axis=1, keepdims=True)
                out[b, start:start + len(r), h, :] = p @ v[b, :, g, :]
    return out
