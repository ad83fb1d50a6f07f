"""Pins for the oracle's visibility mask, tile classification, ring slot and RoPE.

Each test checks the oracle against something other than its own formula: a
closed-form count, the plain causal mask, a structural property, or the
complex-number form of the rotation.
"""
import itertools

import numpy as np
import pytest

import oracle


CASES = [(T, M, W) for T in (1, 2, 5, 17, 64) for M in (0, 1, 4, 8) for W in (-1, 0, 1, 2, 3, 16, 63, 64, 65)
         if M <= T]


@pytest.mark.parametrize("T,M,W", CASES)
def test_mask_row_counts_closed_form(T, M, W):
    # Row i sees its M meta keys plus the last W real keys: min(i+1, M+W);
    # without a window, every earlier key: i+1.
    m = oracle.mask(T, M, W)
    i = np.arange(T)
    expect = i + 1 if W <= 0 else np.minimum(i + 1, M + W)
    assert np.array_equal(m.sum(axis=1), expect)
    assert int(m.sum()) == int(expect.sum())


@pytest.mark.parametrize("T,M,W", CASES)
def test_visible_count_closed_form_and_brute_force(T, M, W):
    # visible_count against (1) the closed form min(i+1, M+W) (i+1 without a
    # window) and (2) row sums of the scalar predicate enumerated pair by pair
    got = oracle.visible_count(T, M, W)
    i = np.arange(T)
    closed = i + 1 if W <= 0 else np.minimum(i + 1, M + W)
    assert got.shape == (T,)
    assert np.array_equal(got, closed)
    brute = [sum(1 for j in range(T) if oracle.visible(r, j, M, W)) for r in range(T)]
    assert np.array_equal(got, np.array(brute))


def test_visible_count_planted_mistakes_fail():
    # the closed form distinguishes the plausible mistakes: a window counted
    # without the row itself, meta keys counted twice, or the count taken
    # over the key axis (column sums)
    T, M, W = 40, 4, 8
    got = oracle.visible_count(T, M, W)
    i = np.arange(T)
    assert not np.array_equal(got, np.minimum(i, M + W - 1) + 1 - (i >= M + W - 1))
    assert not np.array_equal(got, np.minimum(i + 1, M + W) + np.minimum(i + 1, M))
    assert not np.array_equal(got, oracle.mask(T, M, W).sum(axis=0))


@pytest.mark.parametrize("T,M", [(1, 0), (9, 3), (64, 4), (100, 0)])
def test_window_at_least_length_is_causal(T, M):
    causal = np.tril(np.ones((T, T), dtype=bool))
    for W in (T, T + 1, 10 * T, 0, -5):
        assert np.array_equal(oracle.mask(T, M, W), causal)


@pytest.mark.parametrize("T,M,W", [(64, 4, 16), (40, 8, 1), (33, 1, 3)])
def test_meta_visible_to_every_later_row(T, M, W):
    m = oracle.mask(T, M, W)
    for i in range(T):
        for j in range(min(M, i + 1)):
            assert m[i, j]
        # the row's non-meta keys form one contiguous run ending at the row itself
        nz = np.nonzero(m[i, M:])[0] + M
        if i >= M:
            assert nz.max() == i and np.array_equal(nz, np.arange(nz.min(), i + 1))
            assert len(nz) == min(W, i - M + 1) if W > 0 else len(nz) == i - M + 1
        else:
            assert len(nz) == 0


def test_scalar_predicate_agrees_with_matrix():
    for T, M, W in [(12, 3, 4), (20, 0, 5), (7, 7, 2), (16, 2, 0)]:
        m = oracle.mask(T, M, W)
        brute = np.array([[oracle.visible(i, j, M, W) for j in range(T)] for i in range(T)])
        assert np.array_equal(m, brute)


def test_tile_kinds_causal_closed_form():
    # Global causal mask, square tiles: strictly-lower tiles full, diagonal
    # tiles partial (more than one row), upper tiles empty.
    T, b = 70, 16
    k = oracle.tile_kinds(T, 0, 0, b, b)
    n = -(-T // b)
    for a, c in itertools.product(range(n), range(n)):
        if c < a:
            assert k[a, c] == 2
        elif c == a:
            rows = min(b, T - a * b)
            assert k[a, c] == (2 if rows == 1 else 1)
        else:
            assert k[a, c] == 0


def test_tile_kinds_window_skips_far_tiles():
    T, M, W, b = 256, 32, 32, 32
    k = oracle.tile_kinds(T, M, W, b, b)
    # q tile 7 rows 224..255: meta tile 0 full, window needs keys 193..255
    assert k[7, 0] == 2
    assert list(k[7, 1:6]) == [0, 0, 0, 0, 0]
    assert k[7, 6] == 1 and k[7, 7] == 1


def test_cache_slot_ring():
    M, W = 5, 8
    for n in range(0, 40):
        slots = [oracle.cache_slot(s, M, W) for s in range(max(0, n - W + 1), n + 1)]
        assert len(set(slots)) == len(slots)           # the live window never collides
        assert all(M <= s < M + W for s in slots)
    assert oracle.cache_slot(2048, 128, 1024) == 128
    assert oracle.cache_slot(7, 3, 0) == 10
    with pytest.raises(ValueError):
        oracle.cache_slot(-1, 1, 1)


def _rope_complex(x, pos, base):
    # (x_d + i x_{d+Dh/2}) * exp(i * pos * base^(-2d/Dh))
    Dh = x.shape[-1]
    h = Dh // 2
    z = x[..., :h] + 1j * x[..., h:]
    ang = np.outer(pos, base ** (-np.arange(0, Dh, 2) / Dh))[None, :, None, :]
    r = z * np.exp(1j * ang)
    return np.concatenate([r.real, r.imag], axis=-1)


def test_rope_equals_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 9, 3, 16))
    pos = np.arange(9) + 1000
    assert np.allclose(oracle.rope(x, pos, 10000.0), _rope_complex(x, pos, 10000.0), atol=1e-12)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 6, 2, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(6), 1e4), x)
    r = oracle.rope(x, np.arange(6) * 37, 1e4)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    q, k = rng.standard_normal((2, 64))
    def dot(m, n):
        qa = oracle.rope(q[None, None, None], [m], 1e4)[0, 0, 0]
        ka = oracle.rope(k[None, None, None], [n], 1e4)[0, 0, 0]
        return qa @ ka
    assert abs(dot(10, 3) - dot(1010, 1003)) < 1e-9
    assert abs(dot(16511, 16500) - dot(11, 0)) < 1e-9


def test_rope_hand_worked_fixture():
    """tests/golden/rope_handworked.json: the pairing (d, d + Dh/2) and both
    frequencies, derived by hand."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_handworked.json")))
    x = np.array(fx["x"])[None, None, None]
    got = oracle.rope(x, [fx["position"]], fx["base"])[0, 0, 0]
    np.testing.assert_allclose(got, fx["out"], rtol=0, atol=1e-15)
