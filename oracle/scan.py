"""Selective scan of the SSM heads (Mamba, 16 states per channel).

Source: Hymba blog, "数学表示" §4, Eq. (2): the output weight
alpha_ij = C_i (prod_{k=j+1..i} exp(A Delta_k)) B_j Delta_j.  Its recurrent
form, taken step by step here, is

    h_t = exp(Delta_t * A) * h_{t-1} + (Delta_t * x_t) * B_t
    y_t = C_t . h_t

which unrolls to y_i = sum_{j<=i} alpha_ij x_j exactly.  16 states per
channel: model card "模型架构"; the Chinese news article ("模型架構非常巧妙")
and the Spanish article ("Detalles técnicos") both say 16 SSM states.

Readings:
* A [Di, N] is real and negative, one decay per channel and state; B_t, C_t
  [N] are shared by all channels of a token; Delta_t [Di] is already positive
  (no bias or softplus here).  Discretisation exactly as Eq. (2): exp(Delta A)
  for A and Delta * B for B.
* The skip D * x_t and the gate SiLU(z_t) are not on the pages (Eq. (2) shows a
  bare gate G); the output is y_t = (C_t . h_t + D * x_t) * SiLU(z_t).
* h starts at ``h0`` or zero.
"""
from __future__ import annotations

import numpy as np


def _silu(a):
    return a / (1.0 + np.exp(-a))


def selective_scan(x, delta, A, Bm, Cm, D=None, z=None, h0=None):
    """x, delta, z [B, T, Di]; Bm, Cm [B, T, N]; A [Di, N]; D [Di]; h0 [B, Di, N].

    Returns (y [B, T, Di], h_T [B, Di, N]), float64, sequential over t.
    """
    x = np.asarray(x, dtype=np.float64)
    dl = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    Bsz, T, Di = x.shape
    N = A.shape[1]
    h = np.zeros((Bsz, Di, N)) if h0 is None else np.array(h0, dtype=np.float64)
    Dv = None if D is None else np.asarray(D, dtype=np.float64)
    zz = None if z is None else np.asarray(z, dtype=np.float64)
    y = np.empty((Bsz, T, Di))
    for t in range(T):
        h = np.exp(dl[:, t, :, None] * A[None]) * h \
            + (dl[:, t, :] * x[:, t, :])[:, :, None] * Bm[:, t, None, :]
        yt = np.einsum("bdn,bn->bd", h, Cm[:, t, :])
        if Dv is not None:
            yt = yt + Dv * x[:, t, :]
        if zz is not None:
            yt = yt * _silu(zz[:, t, :])
        y[:, t, :] = yt
    return y, h


def scan_step(x, delta, A, Bm, Cm, D, z, h):
    """One token: x, delta, z [B, Di]; Bm, Cm [B, N]; h [B, Di, N]."""
    y, hn = selective_scan(np.asarray(x)[:, None], np.asarray(delta)[:, None], A,
                           np.asarray(Bm)[:, None], np.asarray(Cm)[:, None], D,
                           None if z is None else np.asarray(z)[:, None], h)
    return y[:, 0], hn
