"""Pins for the oracle's attention (Eq. (1) with GQA, RoPE, window, meta tokens).

Library routine: torch's scaled_dot_product_attention on the CPU in float64
with an explicit boolean mask, RoPE applied as a complex multiplication and
GQA expanded with repeat_interleave. Plus special cases and a hand-worked
fixture.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rope_complex(x, pos, base):
    Dh = x.shape[-1]
    h = Dh // 2
    z = x[..., :h] + 1j * x[..., h:]
    ang = np.outer(pos, base ** (-np.arange(0, Dh, 2) / Dh))[None, :, None, :]
    r = z * np.exp(1j * ang)
    return np.concatenate([r.real, r.imag], axis=-1)


def _sdpa_reference(q, k, v, M, W, base, pos0):
    B, T, Hq, Dh = q.shape
    Hkv = k.shape[2]
    pos = pos0 + np.arange(T)
    qr = torch.from_numpy(_rope_complex(q, pos, base)).permute(0, 2, 1, 3)
    kr = torch.from_numpy(_rope_complex(k, pos, base)).permute(0, 2, 1, 3)
    vv = torch.from_numpy(v).permute(0, 2, 1, 3)
    kr = kr.repeat_interleave(Hq // Hkv, dim=1)
    vv = vv.repeat_interleave(Hq // Hkv, dim=1)
    ii = torch.arange(T)[:, None]
    jj = torch.arange(T)[None, :]
    allowed = jj <= ii
    if W > 0:
        allowed &= (jj < M) | (ii - jj < W)
    o = F.scaled_dot_product_attention(qr, kr, vv, attn_mask=allowed)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,T,Hq,Hkv,Dh,M,W,pos0", [
    (1, 64, 2, 1, 16, 4, 16, 0),
    (2, 37, 4, 2, 8, 3, 5, 0),
    (1, 50, 6, 3, 64, 8, 7, 11),
    (1, 33, 5, 5, 16, 0, 4, 0),
    (1, 20, 3, 1, 16, 2, 0, 0),
])
def test_attention_matches_sdpa(B, T, Hq, Hkv, Dh, M, W, pos0):
    rng = np.random.default_rng(T * 7 + Hq)
    q = rng.standard_normal((B, T, Hq, Dh))
    k = rng.standard_normal((B, T, Hkv, Dh))
    v = rng.standard_normal((B, T, Hkv, Dh))
    got = oracle.attention(q, k, v, M, W, 10000.0, pos0, block=16)
    ref = _sdpa_reference(q, k, v, M, W, 10000.0, pos0)
    assert np.allclose(got, ref, atol=1e-12, rtol=1e-10)


def test_window_ge_length_equals_causal_sdpa():
    rng = np.random.default_rng(3)
    B, T, H, Dh, M = 1, 40, 2, 16, 4
    q, k, v = (rng.standard_normal((B, T, H, Dh)) for _ in range(3))
    got = oracle.attention(q, k, v, M, T, 10000.0)
    qr = torch.from_numpy(_rope_complex(q, np.arange(T), 1e4)).permute(0, 2, 1, 3)
    kr = torch.from_numpy(_rope_complex(k, np.arange(T), 1e4)).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(qr, kr, torch.from_numpy(v).permute(0, 2, 1, 3),
                                         is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_special_cases_first_row_and_constant_keys():
    rng = np.random.default_rng(4)
    B, T, Hq, Hkv, Dh, M, W = 2, 30, 4, 2, 16, 3, 6
    q = rng.standard_normal((B, T, Hq, Dh))
    v = rng.standard_normal((B, T, Hkv, Dh))
    k = rng.standard_normal((B, T, Hkv, Dh))
    o = oracle.attention(q, k, v, M, W)
    for h in range(Hq):
        assert np.allclose(o[:, 0, h], v[:, 0, h // 2], atol=1e-14)
    # zero keys give equal scores at every position: the mean of visible V
    o0 = oracle.attention(q, np.zeros_like(k), v, M, W)
    m = oracle.mask(T, M, W)
    for i in range(T):
        mean = v[:, m[i]].mean(axis=1)            # [B, Hkv, Dh]
        for h in range(Hq):
            assert np.allclose(o0[:, i, h], mean[:, h // 2], atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(5)
    B, T, Hq, Hkv, Dh = 1, 25, 6, 2, 8
    q = rng.standard_normal((B, T, Hq, Dh))
    k = rng.standard_normal((B, T, Hkv, Dh))
    v = rng.standard_normal((B, T, Hkv, Dh))
    a = oracle.attention(q, k, v, 2, 5)
    b = oracle.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 2, 5)
    assert np.allclose(a, b, atol=1e-14)


def test_meta_tokens_attended_everywhere():
    rng = np.random.default_rng(6)
    B, T, H, Dh, M, W = 1, 64, 2, 16, 4, 16
    q, k = rng.standard_normal((2, B, T, H, Dh))
    # V = indicator(j < M) in every coordinate: output = attention mass on meta keys
    v = np.zeros((B, T, H, Dh))
    v[:, :M] = 1.0
    o = oracle.attention(q, k, v, M, W)
    mass = o[..., 0]
    assert (mass > 0).all()
    ref = _sdpa_reference(q, k, v, M, W, 1e4, 0)[..., 0]
    assert np.allclose(mass, ref, atol=1e-12)
    assert np.allclose(mass[:, :M], 1.0)       # meta rows see only meta keys


def test_position_shift_invariance():
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((3, 1, 20, 2, 16))
    a = oracle.attention(q, k, v, 2, 6, pos0=0)
    b = oracle.attention(q, k, v, 2, 6, pos0=5000)
    assert np.allclose(a, b, atol=1e-9)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 40, 4, 16))
    k, v = rng.standard_normal((2, 2, 40, 2, 16))
    full = oracle.attention(q, k, v, 3, 9)
    rows = [39, 0, 17, 3]
    assert np.array_equal(oracle.attention(q, k, v, 3, 9, rows=rows), full[:, rows])


def test_handworked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "attention_handworked.json")))
    q = np.array(g["q"])[None, :, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    o = oracle.attention(q, k, v, g["n_meta"], g["window"], g["rope_base"], 0, g["scale"])
    assert np.allclose(o[0, :, 0, :], np.array(g["o"]), atol=1e-12)
