"""The seeded input generator: determinism, dtype rounding and distributions."""
import hashlib

import numpy as np
import torch

from workloads import (DECODE_PAIR, SWA_PREFILL, TINY, bf16_bits, bf16_round,
                       decode_inputs, prefill_inputs, stack_layer_roles, STACK, with_)


def _digest(d):
    h = hashlib.sha256()
    for k in sorted(d):
        v = d[k]
        if isinstance(v, dict):
            h.update(_digest(v).encode())
        else:
            h.update(k.encode())
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = prefill_inputs(TINY, seed=0)
    b = prefill_inputs(TINY, seed=0)
    c = prefill_inputs(TINY, seed=1)
    assert _digest(a) == _digest(b) != _digest(c)
    small = with_(DECODE_PAIR, B=2, Di=64, Hq=1, cache_slots=8, n_prev=3)
    assert _digest(decode_inputs(small, 0)) == _digest(decode_inputs(small, 0))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties to even
    ref = torch.from_numpy(a).to(torch.bfloat16)
    assert np.array_equal(bf16_round(a), ref.float().numpy())
    assert np.array_equal(bf16_bits(bf16_round(a)), ref.view(torch.int16).numpy().view(np.uint16))


def test_distributions_and_dtypes():
    shape = with_(SWA_PREFILL, N=256, M=16)
    d = prefill_inputs(shape, 0)
    assert d["q"].dtype == np.float32 and np.array_equal(bf16_round(d["q"]), d["q"])
    assert (d["delta"] > 0).all() and abs(np.median(d["delta"]) - 0.127) < 0.01
    assert (d["A"] < 0).all() and d["A"].shape == (shape.Di, 16)
    assert abs(d["x"].std() - 1) < 0.01 and abs(d["conv_w"].std() - 0.5) < 0.02
    t = prefill_inputs(TINY, 0)
    assert t["q"].shape == (1, 64, 2, 16) and t["x"].shape == (1, 64, 32)


def test_stack_roles():
    r = stack_layer_roles(STACK)
    assert [w for w, _ in r].count(0) == 3
    assert r[1] == (1024, 1) and r[2] == (1024, 1) and r[14] == (1024, 13)
    assert r[30] == (1024, 30) and r[29] == (1024, 28)
    producers = {src for _, src in r}
    assert len(producers) == 3 + 14 + 1 and sum(1 for i, (_, s) in enumerate(r) if s != i) == 14
