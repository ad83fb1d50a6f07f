"""Pins of the whole-block oracle (Hymba blog, "Hymba 的整体架构" and "数学表示"
§2, §4, §5; Hymba-1.5B-Base model card, "模型架构").

Each pin checks the oracle against a hand value, a closed form, brute-force
loops or a special case that reduces to an already pinned function, so that a
dropped term, a swapped column block or a missing residual fails one of them.
"""
import math

import numpy as np
import pytest

import oracle

Hq, Hkv, Dh, Ns, K = 2, 1, 4, 3, 4
Di = Hq * Dh
d, F = 6, 10
M, N, B = 2, 7, 2
T = M + N


def _weights(rng, producer=True):
    rows = Hq * Dh + (2 * Hkv * Dh if producer else 0) + 2 * Di
    return {
        "ln1": 1 + 0.1 * rng.standard_normal(d),
        "ln2": 1 + 0.1 * rng.standard_normal(d),
        "w_in": rng.standard_normal((rows, d)) / math.sqrt(d),
        "w_dbc": rng.standard_normal((Di + 2 * Ns, Di)) / math.sqrt(Di),
        "dt_bias": -1 + 0.1 * rng.standard_normal(Di),
        "A": -np.exp(0.5 * rng.standard_normal((Di, Ns))),
        "D": rng.standard_normal(Di),
        "conv_w": rng.standard_normal((Di, K)) / 2,
        "conv_b": 0.1 * rng.standard_normal(Di),
        "beta_a": 1 + 0.1 * rng.standard_normal(Di),
        "beta_s": 1 + 0.1 * rng.standard_normal(Di),
        "w_out": rng.standard_normal((d, Di)) / math.sqrt(Di),
        "w_up": rng.standard_normal((F, d)) / math.sqrt(d),
        "w_down": rng.standard_normal((d, F)) / math.sqrt(F),
    }


def test_rms_norm_hand_value():
    # x = (3, 4): mean square 12.5
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y, [3 / r, 8 / r], rtol=1e-15)
    # eps enters under the root
    y = oracle.rms_norm(np.array([1.0, 1.0]), np.ones(2), eps=3.0)
    np.testing.assert_allclose(y, [0.5, 0.5], rtol=1e-15)


def test_silu_and_softplus_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert abs(oracle.softplus(0.0) - math.log(2.0)) < 1e-15
    x = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle.softplus(x) - oracle.softplus(-x), x, atol=1e-12)
    assert oracle.softplus(1000.0) == 1000.0
    assert 0 < oracle.softplus(-700.0) < 1e-300


def test_ffn_brute_force():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((3, d))
    wu = rng.standard_normal((F, d))
    wd = rng.standard_normal((d, F))
    y = oracle.ffn(u, wu, wd)
    for r in range(3):
        a = [sum(wu[f, i] * u[r, i] for i in range(d)) for f in range(F)]
        a = [t / (1 + math.exp(-t)) for t in a]
        for o in range(d):
            assert abs(y[r, o] - sum(wd[o, f] * a[f] for f in range(F))) < 1e-12


def test_zero_output_weights_leave_hidden_unchanged():
    rng = np.random.default_rng(4)
    p = _weights(rng)
    p["w_out"] = np.zeros_like(p["w_out"])
    p["w_down"] = np.zeros_like(p["w_down"])
    h = rng.standard_normal((B, T, d))
    r = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 4)
    np.testing.assert_array_equal(r["hidden"], h)
    np.testing.assert_array_equal(r["mid"], h)


def _mixer_inputs_by_loops(h, p, producer=True, eps=1e-6):
    """The block's mixer inputs, row by row with explicit sums."""
    q = np.zeros((B, T, Hq * Dh)); k = np.zeros((B, T, Hkv * Dh)); v = np.zeros((B, T, Hkv * Dh))
    x = np.zeros((B, T, Di)); z = np.zeros((B, T, Di)); dl = np.zeros((B, T, Di))
    Bm = np.zeros((B, T, Ns)); Cm = np.zeros((B, T, Ns))
    W = p["w_in"]
    for b in range(B):
        for t in range(T):
            ms = sum(h[b, t, i] ** 2 for i in range(d)) / d
            u = [h[b, t, i] / math.sqrt(ms + eps) * p["ln1"][i] for i in range(d)]
            row = [sum(W[o, i] * u[i] for i in range(d)) for o in range(W.shape[0])]
            o = 0
            for dst in ((q, k, v, x, z) if producer else (q, x, z)):
                n = dst.shape[2]
                dst[b, t] = row[o:o + n]
                o += n
            assert o == W.shape[0]
            for c in range(Di):
                a = sum(p["w_dbc"][c, i] * x[b, t, i] for i in range(Di)) + p["dt_bias"][c]
                dl[b, t, c] = math.log1p(math.exp(a))
            for s in range(Ns):
                Bm[b, t, s] = sum(p["w_dbc"][Di + s, i] * x[b, t, i] for i in range(Di))
                Cm[b, t, s] = sum(p["w_dbc"][Di + Ns + s, i] * x[b, t, i] for i in range(Di))
    inp = {"q": q.reshape(B, T, Hq, Dh), "k": k.reshape(B, T, Hkv, Dh),
           "v": v.reshape(B, T, Hkv, Dh), "x": x, "delta": dl, "Bm": Bm, "Cm": Cm, "z": z}
    for key in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s"):
        inp[key] = p[key]
    return inp


def test_mixer_half_matches_loops_and_the_pinned_mixer():
    """With W_down = 0 the block adds W_out mixer(norm1(h)) to h; the mixer's
    inputs are rebuilt by loops and fed to the (separately pinned) mixer."""
    rng = np.random.default_rng(5)
    p = _weights(rng)
    p["w_down"] = np.zeros_like(p["w_down"])
    h = rng.standard_normal((B, T, d))
    r = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 4)
    mo = oracle.mixer_prefill(_mixer_inputs_by_loops(h, p), M, 4)["out"]
    np.testing.assert_allclose(r["mixer_out"], mo, rtol=1e-12, atol=1e-12)
    for b in range(B):
        for t in range(T):
            for o in range(d):
                ref = h[b, t, o] + sum(p["w_out"][o, c] * mo[b, t, c] for c in range(Di))
                assert abs(r["hidden"][b, t, o] - ref) < 1e-12


def test_ffn_half_is_residual_prenorm():
    """With W_out = 0 the block is h + W_down SiLU(W_up norm2(h))."""
    rng = np.random.default_rng(6)
    p = _weights(rng)
    p["w_out"] = np.zeros_like(p["w_out"])
    h = rng.standard_normal((B, T, d))
    r = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 0)
    for b in range(B):
        for t in range(T):
            ms = sum(h[b, t, i] ** 2 for i in range(d)) / d
            u = [h[b, t, i] / math.sqrt(ms + 1e-6) * p["ln2"][i] for i in range(d)]
            a = [sum(p["w_up"][f, i] * u[i] for i in range(d)) for f in range(F)]
            a = [s / (1 + math.exp(-s)) for s in a]
            for o in range(d):
                ref = h[b, t, o] + sum(p["w_down"][o, f] * a[f] for f in range(F))
                assert abs(r["hidden"][b, t, o] - ref) < 1e-12


def test_consumer_block_uses_the_producer_kv():
    """A consumer with the producer's Q, x, z rows and its K, V reproduces the
    producer block exactly (so the consumer's column order is Q, x, z)."""
    rng = np.random.default_rng(7)
    p = _weights(rng)
    h = rng.standard_normal((B, T, d))
    prod = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 3)
    c = dict(p)
    qd, kd = Hq * Dh, Hkv * Dh
    c["w_in"] = np.concatenate([p["w_in"][:qd], p["w_in"][qd + 2 * kd:]], axis=0)
    cons = oracle.block_prefill(h, c, Hq, Hkv, Dh, M, 3, kv=(prod["k"], prod["v"]))
    np.testing.assert_array_equal(cons["hidden"], prod["hidden"])
    # and different K, V change it
    other = oracle.block_prefill(h, c, Hq, Hkv, Dh, M, 3, kv=(prod["k"] * 2, prod["v"]))
    assert np.abs(other["hidden"] - prod["hidden"]).max() > 1e-3


def test_consumer_loops():
    """The consumer's mixer inputs by loops over its 3-block in-projection."""
    rng = np.random.default_rng(8)
    p = _weights(rng, producer=False)
    p["w_down"] = np.zeros_like(p["w_down"])
    h = rng.standard_normal((B, T, d))
    kv = (rng.standard_normal((B, T, Hkv, Dh)), rng.standard_normal((B, T, Hkv, Dh)))
    r = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 4, kv=kv)
    inp = _mixer_inputs_by_loops(h, p, producer=False)
    inp["k"], inp["v"] = kv
    mo = oracle.mixer_prefill(inp, M, 4)["out"]
    np.testing.assert_allclose(r["mixer_out"], mo, rtol=1e-12, atol=1e-12)


def test_stack_chains_blocks_and_shares_kv():
    rng = np.random.default_rng(9)
    roles = [(0, 0), (4, 1), (4, 1), (0, 3)]
    layers = [_weights(rng, producer=(src == l)) for l, (_, src) in enumerate(roles)]
    h = rng.standard_normal((B, T, d))
    r = oracle.stack_prefill(h, layers, roles, Hq, Hkv, Dh, M)
    x = h
    kv1 = None
    for l, (w, src) in enumerate(roles):
        o = oracle.block_prefill(x, layers[l], Hq, Hkv, Dh, M, w, kv=kv1 if src != l else None)
        if l == 1:
            kv1 = (o["k"], o["v"])
        np.testing.assert_array_equal(r["per_layer"][l], o["hidden"])
        x = o["hidden"]
    np.testing.assert_array_equal(r["hidden"], x)


def test_meta_rows_do_not_see_tokens():
    """Through a whole block the meta rows (and every row i) depend only on
    rows <= i: changing the last token leaves all earlier rows unchanged."""
    rng = np.random.default_rng(10)
    p = _weights(rng)
    h = rng.standard_normal((B, T, d))
    r0 = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 3)["hidden"]
    h2 = h.copy()
    h2[:, -1] += 1.0
    r1 = oracle.block_prefill(h2, p, Hq, Hkv, Dh, M, 3)["hidden"]
    np.testing.assert_array_equal(r0[:, :-1], r1[:, :-1])
    assert np.abs(r0[:, -1] - r1[:, -1]).max() > 1e-3


def test_whole_block_by_loops():
    """Both halves at once: the FFN's norm reads h1 = h + W_out mixer(...)."""
    rng = np.random.default_rng(11)
    p = _weights(rng)
    h = rng.standard_normal((B, T, d))
    r = oracle.block_prefill(h, p, Hq, Hkv, Dh, M, 4)
    mo = oracle.mixer_prefill(_mixer_inputs_by_loops(h, p), M, 4)["out"]
    for b in range(B):
        for t in range(T):
            h1 = [h[b, t, o] + sum(p["w_out"][o, c] * mo[b, t, c] for c in range(Di))
                  for o in range(d)]
            ms = sum(v * v for v in h1) / d
            u = [h1[i] / math.sqrt(ms + 1e-6) * p["ln2"][i] for i in range(d)]
            a = [sum(p["w_up"][f, i] * u[i] for i in range(d)) for f in range(F)]
            a = [s / (1 + math.exp(-s)) for s in a]
            for o in range(d):
                ref = h1[o] + sum(p["w_down"][o, f] * a[f] for f in range(F))
                assert abs(r["mid"][b, t, o] - h1[o]) < 1e-12
                assert abs(r["hidden"][b, t, o] - ref) < 1e-12
