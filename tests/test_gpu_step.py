"""GPU parity of the decode step (one token, a KV-sharing pair of layers).

Producer then consumer on one shared cache, compared with the oracle's step on
the same inputs: output, both branch outputs, the advanced conv/SSM states and
the cache row the producer writes.
"""
import numpy as np
import pytest

import oracle
from workloads import DECODE_PAIR, TINY, decode_inputs, with_

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import assert_close, down, up_inputs  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_pair(shape, seed, scale=0.0):
    d = decode_inputs(shape, seed)
    t = up_inputs(d, shape.dtype)
    kc, vc = t["k_cache"], t["v_cache"]
    pa = hm.StepPlan(t["a"], kc, vc, shape.n_prev, shape.M, shape.W, rope_base=shape.rope_base,
                     eps=shape.eps, scale=scale, want_branches=True)
    pb = hm.StepPlan(t["b"], kc, vc, shape.n_prev, shape.M, shape.W, rope_base=shape.rope_base,
                     eps=shape.eps, scale=scale, want_branches=True)
    pa.run()
    pb.run()
    torch.cuda.synchronize()
    ra = oracle.mixer_step(d["a"], d["k_cache"], d["v_cache"], shape.n_prev, shape.M, shape.W,
                           producer=True, rope_base=shape.rope_base, eps=shape.eps, scale=scale)
    rb = oracle.mixer_step(d["b"], ra["k_cache"], ra["v_cache"], shape.n_prev, shape.M, shape.W,
                           producer=False, rope_base=shape.rope_base, eps=shape.eps, scale=scale)
    return d, t, (pa, pb), (ra, rb)


def _check(shape, seed, scale=0.0):
    d, t, plans, refs = _run_pair(shape, seed, scale)
    dt = shape.dtype
    for name, plan, ref in zip("ab", plans, refs):
        assert_close(down(plan.out), ref["out"], dt, f"{name} out")
        assert_close(down(plan.ya), ref["ya"], dt, f"{name} ya")
        assert_close(down(plan.ys), ref["ys"], dt, f"{name} ys")
        assert_close(down(t[name]["ssm_state"]), ref["ssm_state"], dt, f"{name} ssm_state")
        assert np.array_equal(down(t[name]["conv_state"]), ref["conv_state"]), f"{name} conv"
    slot = oracle.cache_slot(shape.n_prev, shape.M, shape.W)
    assert hm.debug_cache_slot(shape.n_prev, shape.M, shape.W) == slot
    kc = down(t["k_cache"])
    vc = down(t["v_cache"])
    assert_close(kc[:, slot], refs[0]["k_cache"][:, slot], dt, "written K row")
    assert np.array_equal(vc[:, slot], refs[0]["v_cache"][:, slot])
    # every other row is untouched
    others = [r for r in range(kc.shape[1]) if r != slot]
    assert np.array_equal(kc[:, others], d["k_cache"][:, others].astype(np.float64))



# a caller's softmax scale and another RoPE base (the cache built with that base)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_scale_and_rope_base(dtype):
    shape = with_(DECODE_PAIR, B=3, n_prev=1700, rope_base=500000.0, dtype=dtype)
    if dtype == "f32":
        shape = with_(shape, Hq=4, Hkv=2, Dh=32, Di=128)
    _check(shape, 9, scale=0.2)

def test_decode_pair_full_size():
    _check(DECODE_PAIR, 0)


@pytest.mark.parametrize("n_prev", [0, 1, 63, 64, 300, 1023, 1024, 1025, 5000])
def test_decode_pair_bf16_window_positions(n_prev):
    shape = with_(DECODE_PAIR, B=3, n_prev=n_prev)
    _check(shape, n_prev)


@pytest.mark.parametrize("n_prev", [0, 5, 200])
def test_decode_pair_bf16_global(n_prev):
    shape = with_(DECODE_PAIR, B=2, W=0, cache_slots=256, n_prev=n_prev, M=30)
    _check(shape, 11 + n_prev)


@pytest.mark.parametrize("M,W,n_prev", [(5, 100, 0), (5, 100, 99), (5, 100, 100), (5, 100, 350),
                                         (63, 65, 64), (1, 127, 500)])
def test_decode_pair_bf16_unaligned_window(M, W, n_prev):
    """Meta and window lengths off the 64-row tile grid: the visible rows end
    inside a tile, and the ring slot wraps at a window that is not a tile
    multiple."""
    shape = with_(DECODE_PAIR, B=4, M=M, W=W, cache_slots=W, n_prev=n_prev)
    _check(shape, 31 + n_prev)


def test_decode_pair_bf16_global_long_cache():
    """A global layer with a long cache: more key splits than the combine keeps
    in registers."""
    shape = with_(DECODE_PAIR, B=2, W=0, cache_slots=4096, n_prev=3000, M=64)
    _check(shape, 17)


@pytest.mark.parametrize("n_prev", [6000, 16384])
def test_decode_pair_bf16_global_single_sequence(n_prev):
    """One sequence through a global layer with a long cache: the most key
    splits per (sequence, KV head), capped so that the combine holds every
    (query head, split) pair (the stack's global layers at 16 K context)."""
    shape = with_(DECODE_PAIR, B=1, W=0, cache_slots=16512, n_prev=n_prev, M=128)
    _check(shape, 23)


@pytest.mark.parametrize("B,n_prev,M,W", [(64, 2048, 128, 1024), (5, 0, 4, 16), (7, 999, 3, 0),
                                          (130, 5000, 128, 1024)])
def test_step_positions_bit_exact(B, n_prev, M, W):
    """Slot, visible rows and position of every sequence, from the decode
    kernels' own device function, against the oracle's ring slot and valid
    slot set; uniform and ragged batches (entries past n_prev and below zero
    clamped)."""
    rng = np.random.default_rng(B + n_prev)
    for ragged in (False, True):
        nps = None
        if ragged:
            nps = rng.integers(-3, n_prev + 4, size=B).astype(np.int32)
        got = hm.debug_step_positions(B, n_prev, M, W,
                                      None if nps is None else torch.from_numpy(nps).cuda())
        got = got.cpu().numpy()
        for b in range(B):
            npb = n_prev if nps is None else int(min(max(nps[b], 0), n_prev))
            slot = oracle.cache_slot(npb, M, W)
            valid = oracle.valid_slots(npb, M, W)
            assert got[b, 0] == slot, (b, npb)
            # the kernels read rows 0 .. L-1: exactly the valid slots
            assert np.array_equal(valid, np.arange(got[b, 1])), (b, npb)
            assert got[b, 2] == M + npb


@pytest.mark.parametrize("n_prev", [0, 5, 15, 16, 40])
@pytest.mark.parametrize("Dh", [16, 64])
def test_decode_pair_f32(n_prev, Dh):
    shape = with_(TINY, B=2, n_prev=n_prev, cache_slots=16, Dh=Dh, Di=2 * Dh)
    _check(shape, 3)


def test_decode_repeated_calls_reuse_workspace():
    """Three tokens in a row through the same plans (same workspace, states
    advancing in place) against the oracle stepped three times."""
    shape = with_(DECODE_PAIR, B=4, n_prev=700)
    d = decode_inputs(shape, 5)
    t = up_inputs(d, shape.dtype)
    pa = hm.StepPlan(t["a"], t["k_cache"], t["v_cache"], shape.n_prev, shape.M, shape.W)
    pb = hm.StepPlan(t["b"], t["k_cache"], t["v_cache"], shape.n_prev, shape.M, shape.W)
    la, lb = dict(d["a"]), dict(d["b"])
    kc, vc = d["k_cache"], d["v_cache"]
    for it in range(3):
        pa.run()
        pb.run()
        torch.cuda.synchronize()
        ra = oracle.mixer_step(la, kc, vc, shape.n_prev, shape.M, shape.W, producer=True)
        rb = oracle.mixer_step(lb, ra["k_cache"], ra["v_cache"], shape.n_prev, shape.M, shape.W,
                               producer=False)
        assert_close(down(pa.out), ra["out"], "bf16", f"producer out, call {it}")
        assert_close(down(pb.out), rb["out"], "bf16", f"consumer out, call {it}")
        la["conv_state"], la["ssm_state"] = ra["conv_state"], ra["ssm_state"]
        lb["conv_state"], lb["ssm_state"] = rb["conv_state"], rb["ssm_state"]
        kc, vc = ra["k_cache"], ra["v_cache"]
    assert_close(down(t["a"]["ssm_state"]), la["ssm_state"], "bf16", "state after 3 calls")


def test_decode_pair_shared_garbage_workspace():
    """Producer and consumer share one workspace that starts out as random
    bytes (no part of it may need clearing); the batch of 3 makes the SSM
    shares of workgroups straddle sequences.  Two calls in a row."""
    shape = with_(DECODE_PAIR, B=3, n_prev=333)
    d = decode_inputs(shape, 8)
    t = up_inputs(d, shape.dtype)
    gen = torch.Generator(device="cpu").manual_seed(4)
    probe = hm.StepPlan(t["a"], t["k_cache"], t["v_cache"], shape.n_prev, shape.M, shape.W)
    nb = probe.ws.numel()
    ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, generator=gen).to("cuda")
    pa = hm.StepPlan(t["a"], t["k_cache"], t["v_cache"], shape.n_prev, shape.M, shape.W,
                     workspace=ws)
    pb = hm.StepPlan(t["b"], t["k_cache"], t["v_cache"], shape.n_prev, shape.M, shape.W,
                     workspace=ws)
    la, lb = dict(d["a"]), dict(d["b"])
    kc, vc = d["k_cache"], d["v_cache"]
    for it in range(2):
        pa.run()
        pb.run()
        torch.cuda.synchronize()
        ra = oracle.mixer_step(la, kc, vc, shape.n_prev, shape.M, shape.W, producer=True)
        rb = oracle.mixer_step(lb, ra["k_cache"], ra["v_cache"], shape.n_prev, shape.M, shape.W,
                               producer=False)
        assert_close(down(pa.out), ra["out"], "bf16", f"producer out, call {it}")
        assert_close(down(pb.out), rb["out"], "bf16", f"consumer out, call {it}")
        la["conv_state"], la["ssm_state"] = ra["conv_state"], ra["ssm_state"]
        lb["conv_state"], lb["ssm_state"] = rb["conv_state"], rb["ssm_state"]
        kc, vc = ra["k_cache"], ra["v_cache"]


def _check_ragged(shape, nps, seed):
    """Producer then consumer with one n_prev per sequence, against the
    oracle's ragged step."""
    d = decode_inputs(shape, seed)
    t = up_inputs(d, shape.dtype)
    kc, vc = t["k_cache"], t["v_cache"]
    npt = torch.tensor(nps, dtype=torch.int32, device="cuda")
    plans = [hm.StepPlan(t[name], kc, vc, shape.n_prev, shape.M, shape.W, want_branches=True,
                         n_prev_seq=npt) for name in "ab"]
    for p in plans:
        p.run()
    torch.cuda.synchronize()
    ra = oracle.mixer_step_ragged(d["a"], d["k_cache"], d["v_cache"], nps, shape.M, shape.W,
                                  producer=True)
    rb = oracle.mixer_step_ragged(d["b"], ra["k_cache"], ra["v_cache"], nps, shape.M, shape.W,
                                  producer=False)
    dt = shape.dtype
    for name, plan, ref in zip("ab", plans, (ra, rb)):
        assert_close(down(plan.out), ref["out"], dt, f"{name} out")
        assert_close(down(plan.ya), ref["ya"], dt, f"{name} ya")
        assert_close(down(plan.ys), ref["ys"], dt, f"{name} ys")
        assert_close(down(t[name]["ssm_state"]), ref["ssm_state"], dt, f"{name} ssm_state")
    kcd = down(kc)
    for b, npb in enumerate(nps):
        slot = oracle.cache_slot(int(npb), shape.M, shape.W)
        assert_close(kcd[b, slot], ra["k_cache"][b, slot], dt, f"written K row of sequence {b}")
    # rows other than each sequence's own slot are untouched
    for b, npb in enumerate(nps):
        slot = oracle.cache_slot(int(npb), shape.M, shape.W)
        others = [r for r in range(kcd.shape[1]) if r != slot]
        assert np.array_equal(kcd[b, others], d["k_cache"][b, others].astype(np.float64))


def test_decode_pair_bf16_ragged_window():
    """Sequences before, at and after the ring wraps, in one batch."""
    shape = with_(DECODE_PAIR, B=5, n_prev=3000)
    _check_ragged(shape, [0, 63, 700, 1024, 3000], 31)


def test_decode_pair_bf16_ragged_global():
    shape = with_(DECODE_PAIR, B=3, W=0, cache_slots=256, n_prev=200, M=30)
    _check_ragged(shape, [0, 5, 200], 32)


@pytest.mark.parametrize("Dh", [16, 64])
def test_decode_pair_f32_ragged(Dh):
    shape = with_(TINY, B=3, n_prev=40, cache_slots=16, Dh=Dh, Di=2 * Dh)
    _check_ragged(shape, [0, 15, 40], 33)


@pytest.mark.parametrize("n_prev,W", [(150, 64), (40, 0)])
def test_prefill_states_feed_the_decode_step(n_prev, W):
    """The SSM-branch states a GPU prefill returns (conv_state_out, h_out) drive
    a GPU decode step for the next token: its output equals the last row of an
    oracle prefill over one more row.  The cache comes from the oracle."""
    from workloads import SWA_PREFILL, bf16_round, prefill_inputs
    shape = with_(SWA_PREFILL, B=2, M=8, N=n_prev + 1, Hq=4, Hkv=2, Di=256, W=W)
    M, T = shape.M, shape.M + n_prev            # prefill rows; the decode token is row T
    full = prefill_inputs(shape, 21)
    rows = ("q", "k", "v", "x", "delta", "Bm", "Cm", "z")
    pre = {k: (np.ascontiguousarray(full[k][:, :T]) if k in rows else full[k]) for k in full}
    t = up_inputs(pre, "bf16")
    plan = hm.PrefillPlan(t, M, W, rope_base=shape.rope_base, eps=shape.eps, want_states=True)
    plan.run()
    slots = W if W > 0 else n_prev + 1
    kc, vc = oracle.build_cache(full["k"], full["v"], M, n_prev, W, slots, shape.rope_base, fill=0.0)
    step = {"q": full["q"][:, T], "k_new": full["k"][:, T], "v_new": full["v"][:, T]}
    for k in ("x", "delta", "Bm", "Cm", "z"):
        step[k] = full[k][:, T]
    step = up_inputs(step, "bf16")
    for k in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s"):
        step[k] = t[k]
    step["conv_state"], step["ssm_state"] = plan.conv_state, plan.h     # GPU prefill -> decode
    kcd = up_inputs({"k_cache": bf16_round(kc)}, "bf16")["k_cache"]
    vcd = up_inputs({"v_cache": bf16_round(vc)}, "bf16")["v_cache"]
    sp = hm.StepPlan(step, kcd, vcd, n_prev, M, W, rope_base=shape.rope_base, eps=shape.eps)
    sp.run()
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill(full, M, W, shape.rope_base, shape.eps)["out"][:, T]
    assert_close(down(sp.out), ref, "bf16", "decode after prefill")
