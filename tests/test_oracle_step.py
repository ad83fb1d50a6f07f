"""Pins for the oracle's decode step against its prefill (a second formulation).

After prefill over M + t rows, one decode step for the token at position
M + t must give the same output as the last row of prefill over M + t + 1
rows, for the producer (writes its K/V into the ring) and for the consumer
(reads the producer's K/V with its own q).
"""
import numpy as np
import pytest

import oracle
from workloads import TINY, prefill_inputs, with_


def _split(inp, L):
    return {k: (v[:, :L] if k in ("q", "k", "v", "x", "delta", "Bm", "Cm", "z") else v)
            for k, v in inp.items()}


@pytest.mark.parametrize("t", [0, 1, 5, 15, 16, 17, 40, 59])
@pytest.mark.parametrize("window", [16, 0])
def test_decode_step_equals_last_prefill_row(t, window):
    shape = with_(TINY, W=window)
    inp = prefill_inputs(shape, seed=21)
    M = shape.M
    slots = 60 if window <= 0 else window
    full = oracle.mixer_prefill(_split(inp, M + t + 1), M, window)
    prev = oracle.mixer_prefill(_split(inp, M + t), M, window) if M + t > 0 else None
    kc, vc = oracle.build_cache(inp["k"], inp["v"], M, t, window, slots, fill=np.nan)
    layer = {
        "q": inp["q"][:, M + t], "k_new": inp["k"][:, M + t], "v_new": inp["v"][:, M + t],
        "x": inp["x"][:, M + t], "delta": inp["delta"][:, M + t], "Bm": inp["Bm"][:, M + t],
        "Cm": inp["Cm"][:, M + t], "z": inp["z"][:, M + t],
        "conv_state": prev["conv_state"], "ssm_state": prev["ssm_state"],
    }
    for k in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s"):
        layer[k] = inp[k]
    r = oracle.mixer_step(layer, kc, vc, t, M, window, producer=True)
    assert np.allclose(r["out"], full["out"][:, -1], atol=1e-12)
    assert np.allclose(r["ya"], full["ya"][:, -1], atol=1e-12)
    assert np.allclose(r["ys"], full["ys"][:, -1], atol=1e-12)
    assert np.allclose(r["ssm_state"], full["ssm_state"], atol=1e-12)
    assert np.allclose(r["conv_state"], full["conv_state"], atol=1e-14)
    # the cache after the write equals the cache built from prefill over t+1 tokens
    kc2, vc2 = oracle.build_cache(inp["k"], inp["v"], M, t + 1, window, slots, fill=np.nan)
    rows = oracle.valid_slots(t, M, window)
    assert np.allclose(r["k_cache"][:, rows], kc2[:, rows], atol=1e-12)
    assert np.array_equal(r["v_cache"][:, rows], vc2[:, rows])


@pytest.mark.parametrize("t", [3, 30])
def test_consumer_reads_producer_cache(t):
    shape = TINY
    M, W = shape.M, shape.W
    prod = prefill_inputs(shape, seed=31)
    cons = prefill_inputs(shape, seed=32)
    # consumer layer: own q / SSM inputs, producer's K and V
    mixed = dict(cons)
    mixed["k"], mixed["v"] = prod["k"], prod["v"]
    full = oracle.mixer_prefill(_split(mixed, M + t + 1), M, W)
    prev = oracle.mixer_prefill(_split(mixed, M + t), M, W)
    kc, vc = oracle.build_cache(prod["k"], prod["v"], M, t + 1, W, W, fill=np.nan)
    layer = {k: cons[k][:, M + t] for k in ("q", "x", "delta", "Bm", "Cm", "z")}
    layer.update({k: cons[k] for k in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s")})
    layer["conv_state"], layer["ssm_state"] = prev["conv_state"], prev["ssm_state"]
    r = oracle.mixer_step(layer, kc, vc, t, M, W, producer=False)
    assert np.allclose(r["out"], full["out"][:, -1], atol=1e-12)
    assert np.array_equal(np.nan_to_num(r["k_cache"], nan=7.0), np.nan_to_num(kc, nan=7.0))


def test_valid_slots_counts():
    for n in range(0, 50):
        s = oracle.valid_slots(n, 4, 16)
        assert len(s) == 4 + min(n + 1, 16) and len(set(s.tolist())) == len(s)
        assert oracle.cache_slot(n, 4, 16) in s
    s = oracle.valid_slots(9, 2, 0)
    assert s.tolist() == list(range(2 + 10))


def test_ragged_step_equals_uniform_steps():
    """A ragged batch (one n_prev per sequence) gives each sequence exactly the
    step of a uniform batch at its n_prev, and a uniform n_prev_seq equals the
    scalar step."""
    from workloads import DECODE_PAIR, decode_inputs
    shape = with_(DECODE_PAIR, B=3, Hq=4, Hkv=2, Dh=16, Di=64, M=3, W=8, cache_slots=8,
                  n_prev=20, dtype="f32")
    d = decode_inputs(shape, 2)
    nps = np.array([0, 7, 20])
    rag = oracle.mixer_step_ragged(d["a"], d["k_cache"], d["v_cache"], nps, shape.M, shape.W,
                                   producer=True)
    for b, npb in enumerate(nps):
        ref = oracle.mixer_step(d["a"], d["k_cache"], d["v_cache"], int(npb), shape.M, shape.W,
                                producer=True)
        for key in ("out", "ya", "ys", "conv_state", "ssm_state", "k_cache", "v_cache"):
            np.testing.assert_allclose(rag[key][b], ref[key][b], rtol=1e-13, atol=1e-13,
                                       err_msg=key)
    uni = oracle.mixer_step_ragged(d["a"], d["k_cache"], d["v_cache"], np.full(3, 5), shape.M,
                                   shape.W, producer=True)
    ref = oracle.mixer_step(d["a"], d["k_cache"], d["v_cache"], 5, shape.M, shape.W,
                            producer=True)
    for key in ("out", "k_cache"):
        np.testing.assert_allclose(uni[key], ref[key], rtol=1e-13, atol=1e-13)
