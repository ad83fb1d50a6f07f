"""Pins for the oracle's causal conv1d, selective scan (Eq. (2)) and norm-and-average.

Library routines (torch conv1d, scipy lfilter, torch rms_norm), the quadratic
form of Eq. (2) by brute force, closed forms, state hand-off and hand-worked
fixtures.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _silu(a):
    return a / (1 + np.exp(-a))


# ---------------------------------------------------------------- conv
@pytest.mark.parametrize("B,T,Di,K", [(1, 64, 32, 4), (2, 3, 5, 4), (1, 17, 7, 2), (3, 1, 4, 4)])
def test_conv_matches_torch_conv1d(B, T, Di, K):
    rng = np.random.default_rng(B * 100 + T)
    x = rng.standard_normal((B, T, Di))
    w = rng.standard_normal((Di, K))
    b = rng.standard_normal(Di)
    y, st = oracle.causal_conv1d(x, w, b, None, True)
    ref = F.conv1d(torch.from_numpy(x).permute(0, 2, 1), torch.from_numpy(w)[:, None, :],
                   torch.from_numpy(b), padding=K - 1, groups=Di)[..., :T]
    ref = F.silu(ref).permute(0, 2, 1).numpy()
    assert np.allclose(y, ref, atol=1e-12)
    padded = np.concatenate([np.zeros((B, K - 1, Di)), x], axis=1)
    assert np.array_equal(st, padded[:, -(K - 1):].transpose(0, 2, 1))


def test_conv_impulse_gives_reversed_taps():
    Di, K, T = 3, 4, 8
    w = np.arange(1, Di * K + 1, dtype=float).reshape(Di, K)
    x = np.zeros((1, T, Di))
    x[0, 2] = 1.0
    y, _ = oracle.causal_conv1d(x, w, None, None, False)
    for c in range(Di):
        assert np.array_equal(y[0, 2:2 + K, c], w[c, ::-1])
        assert np.all(y[0, :2, c] == 0) and np.all(y[0, 2 + K:, c] == 0)


def test_conv_state_handoff():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 23, 6))
    w, b = rng.standard_normal((6, 4)), rng.standard_normal(6)
    full, st_full = oracle.causal_conv1d(x, w, b)
    for cut in (1, 2, 3, 10, 22):
        y1, s1 = oracle.causal_conv1d(x[:, :cut], w, b)
        y2, s2 = oracle.causal_conv1d(x[:, cut:], w, b, s1)
        assert np.allclose(np.concatenate([y1, y2], axis=1), full, atol=1e-13)
        assert np.array_equal(s2, st_full)


# ---------------------------------------------------------------- scan
def _scan_quadratic(x, dl, A, Bm, Cm, D, z):
    """Eq. (2) as written: y_i = sum_{j<=i} C_i (prod_{k=j+1..i} exp(A Delta_k)) B_j Delta_j x_j."""
    Bsz, T, Di = x.shape
    N = A.shape[1]
    y = np.zeros((Bsz, T, Di))
    for b in range(Bsz):
        for c in range(Di):
            for i in range(T):
                acc = 0.0
                for j in range(i + 1):
                    for n in range(N):
                        prod = 1.0
                        for k in range(j + 1, i + 1):
                            prod *= math.exp(A[c, n] * dl[b, k, c])
                        acc += Cm[b, i, n] * prod * Bm[b, j, n] * dl[b, j, c] * x[b, j, c]
                y[b, i, c] = (acc + D[c] * x[b, i, c]) * _silu(z[b, i, c])
    return y


def _rand_scan(rng, B, T, Di, N):
    x = rng.standard_normal((B, T, Di))
    dl = np.log1p(np.exp(rng.normal(-2, 0.5, (B, T, Di))))
    A = -np.exp(rng.normal(0, 0.5, (Di, N)))
    Bm, Cm = rng.standard_normal((2, B, T, N))
    D = rng.standard_normal(Di)
    z = rng.standard_normal((B, T, Di))
    return x, dl, A, Bm, Cm, D, z


def test_scan_equals_eq2_quadratic_form():
    rng = np.random.default_rng(10)
    x, dl, A, Bm, Cm, D, z = _rand_scan(rng, 2, 9, 3, 4)
    y, _ = oracle.selective_scan(x, dl, A, Bm, Cm, D, z)
    assert np.allclose(y, _scan_quadratic(x, dl, A, Bm, Cm, D, z), atol=1e-12)


def test_scan_constant_delta_closed_form_and_lfilter():
    # constant Delta = d, x = xi, B = b: h_t = d b xi (1 - a^(t+1)) / (1 - a), a = exp(d A)
    T, Di, N = 50, 3, 16
    rng = np.random.default_rng(11)
    A = -np.exp(rng.normal(0, 0.5, (Di, N)))
    d, xi = 0.13, 0.7
    bvec = rng.standard_normal(N)
    x = np.full((1, T, Di), xi)
    dl = np.full((1, T, Di), d)
    Bm = np.broadcast_to(bvec, (1, T, N)).copy()
    for t_end in (1, 2, 17, 50):
        Cm = np.zeros((1, t_end, N))
        _, h = oracle.selective_scan(x[:, :t_end], dl[:, :t_end], A, Bm[:, :t_end], Cm)
        a = np.exp(d * A)
        closed = d * bvec * xi * (1 - a ** t_end) / (1 - a)
        assert np.allclose(h[0], closed, rtol=1e-12, atol=1e-14)
    # the same recurrence as a first-order IIR filter (library routine)
    c = 1
    u = d * xi * bvec[None, :] * np.ones((T, N))
    for n in range(N):
        a = math.exp(d * A[c, n])
        ref = scipy.signal.lfilter([1.0], [1.0, -a], u[:, n])
        Cm = np.zeros((1, T, N))
        Cm[0, :, n] = 1.0
        y, _ = oracle.selective_scan(x, dl, A, Bm, Cm)
        assert np.allclose(y[0, :, c], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_scan_chunked_equals_sequential(chunk):
    rng = np.random.default_rng(12)
    x, dl, A, Bm, Cm, D, z = _rand_scan(rng, 2, 64, 5, 16)
    y, h = oracle.selective_scan(x, dl, A, Bm, Cm, D, z)
    hc = rng.standard_normal((2, 5, 16)) * 0  # zero start
    ys = []
    for s in range(0, 64, chunk):
        e = min(64, s + chunk)
        yc, hc = oracle.selective_scan(x[:, s:e], dl[:, s:e], A, Bm[:, s:e], Cm[:, s:e], D,
                                       z[:, s:e], hc)
        ys.append(yc)
    assert np.allclose(np.concatenate(ys, axis=1), y, atol=1e-12)
    assert np.allclose(hc, h, atol=1e-12)


def test_scan_degenerate_cases():
    rng = np.random.default_rng(13)
    x, dl, A, Bm, Cm, D, z = _rand_scan(rng, 1, 20, 4, 16)
    y, _ = oracle.selective_scan(x, dl, A, np.zeros_like(Bm), Cm, D, z)
    assert np.allclose(y, D * x * _silu(z), atol=1e-14)
    y, _ = oracle.selective_scan(x, dl, A, Bm, np.zeros_like(Cm), D, z)
    assert np.allclose(y, D * x * _silu(z), atol=1e-14)
    # A -> -inf: no memory, y_t = (C_t . B_t) Delta_t x_t + D x_t, gated
    y, _ = oracle.selective_scan(x, dl, np.full_like(A, -1e6), Bm, Cm, D, z)
    cb = (Cm * Bm).sum(-1)[..., None]
    assert np.allclose(y, (cb * dl * x + D * x) * _silu(z), atol=1e-12)
    # no D, no gate
    y, _ = oracle.selective_scan(x, dl, A, Bm, Cm)
    y2, _ = oracle.selective_scan(x, dl, A, Bm, Cm, np.zeros(4), np.full_like(z, 1e3))
    assert np.allclose(1e3 * y, y2, atol=1e-9)   # SiLU(1000) = 1000


def test_scan_handworked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "scan_handworked.json")))
    x = np.array(g["x"])[None, :, None]
    dl = np.array(g["delta"])[None, :, None]
    y, h = oracle.selective_scan(x, dl, np.array(g["A"]), np.array(g["B"])[None],
                                 np.array(g["C"])[None], np.array(g["D"]))
    assert np.allclose(y[0, :, 0], g["y"], atol=1e-14)
    assert np.allclose(h[0, 0], g["h_final"], atol=1e-14)


# ---------------------------------------------------------------- norm
def test_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(14)
    ya, ys = rng.standard_normal((2, 7, 1600)) * np.array([0.3, 40.0])[:, None, None]
    ba, bs = 1 + 0.1 * rng.standard_normal((2, 1600))
    got = oracle.branch_norm_mean(ya, ys, ba, bs, 1e-6)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    ref = 0.5 * (F.rms_norm(t(ya), (1600,), t(ba), 1e-6) + F.rms_norm(t(ys), (1600,), t(bs), 1e-6))
    assert np.allclose(got, ref.numpy(), atol=1e-12)


def test_norm_invariants():
    rng = np.random.default_rng(15)
    y = rng.standard_normal((5, 32))
    beta = 1 + 0.1 * rng.standard_normal(32)
    r = oracle.rms_normalize(y, 0.0)
    assert np.allclose(np.mean(r * r, axis=-1), 1.0, atol=1e-13)
    assert np.allclose(oracle.branch_norm_mean(y, y, beta, beta, 1e-6),
                       beta * oracle.rms_normalize(y, 1e-6), atol=1e-14)
    assert np.allclose(oracle.branch_norm_mean(y, 1000 * y, beta, beta, 0.0),
                       beta * r, atol=1e-13)


def test_norm_handworked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "norm_handworked.json")))
    out = oracle.branch_norm_mean(np.array(g["ya"]), np.array(g["ys"]), g["beta_a"],
                                  g["beta_s"], g["eps"])
    assert np.allclose(out, g["out"], atol=1e-15)
