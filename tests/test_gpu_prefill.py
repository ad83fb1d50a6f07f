"""GPU parity: the HIP prefill path (through the C ABI) against the CPU oracle.

Tolerances: float32 workloads max|g - r| <= 1e-4 max|r| per output tensor;
bf16-input / fp32-accumulate workloads max|g - r| <= 2e-2 max|r|; the mask,
tile plan and ring slot bit-exact.
"""
import numpy as np
import pytest

import oracle
from workloads import (GLOBAL_PREFILL, SWA_PREFILL, TINY, cached_meta_inputs, prefill_inputs,
                       with_)

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import assert_close, down, up, up_inputs  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ index exports
MASK_CASES = [(64, 4, 16), (1, 0, 0), (2, 1, 1), (100, 0, 7), (130, 128, 0), (300, 16, 100),
              (257, 3, 256), (2176, 128, 1024)]


@pytest.mark.parametrize("T,M,W", MASK_CASES)
def test_mask_bit_exact(T, M, W):
    got = hm.debug_attn_mask(T, M, W).cpu().numpy().astype(bool)
    assert np.array_equal(got, oracle.mask(T, M, W))


TILE_CASES = [(64, 4, 16), (300, 16, 100), (2176, 128, 1024), (8320, 128, 0), (1000, 5, 63),
              (129, 128, 1), (257, 0, 64), (16512, 128, 1024)]


@pytest.mark.parametrize("T,M,W", TILE_CASES)
def test_tile_plan_bit_exact(T, M, W):
    bmw, bmv, bn = hm.debug_attn_tiles()
    for bm, bnn in ((bmw, bn), (bmv, bn), (7, 5), (1, 1) if T <= 300 else (bmw, bn)):
        got = hm.debug_tile_plan(T, M, W, bm, bnn).cpu().numpy()
        assert np.array_equal(got, oracle.tile_kinds(T, M, W, bm, bnn)), (bm, bnn)


# ------------------------------------------------------------------ attention
def _attn_case(shape, seed, rows=None):
    inp = prefill_inputs(shape, seed)
    t = up_inputs(inp, shape.dtype)
    o = hm.swa_meta_attn(t["q"], t["k"], t["v"], shape.M, shape.W, shape.rope_base)
    torch.cuda.synchronize()
    got = down(o)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], shape.M, shape.W, shape.rope_base,
                           rows=rows)
    if rows is not None:
        got = got[:, rows]
    return got, ref


def test_attention_tiny_f32():
    got, ref = _attn_case(TINY, 0)
    assert_close(got, ref, "f32", "attention tiny")


@pytest.mark.parametrize("Dh", [16, 32, 64])
def test_attention_f32_head_dims(Dh):
    shape = with_(TINY, B=2, N=90, Dh=Dh, Hq=4, Hkv=2, W=20, M=6, Di=4 * Dh)
    got, ref = _attn_case(shape, 1)
    assert_close(got, ref, "f32", f"attention f32 Dh={Dh}")


BF16_CASES = [
    # (B, M, N, Hq, Hkv, W): several 128-row query tiles, ragged tails, meta
    # prefixes that end inside a key tile, global and windowed, GQA groups
    (1, 4, 60, 2, 1, 16),
    (2, 16, 284, 10, 2, 100),
    (1, 0, 300, 5, 5, 0),
    (1, 3, 200, 4, 1, 1),
    (1, 128, 2048, 25, 5, 1024),
    (1, 70, 450, 6, 3, 64),
    # every row a meta row (causal among themselves, the window never applies)
    (2, 150, 0, 2, 1, 16),
]


@pytest.mark.parametrize("B,M,N,Hq,Hkv,W", BF16_CASES)
def test_attention_bf16(B, M, N, Hq, Hkv, W):
    shape = with_(SWA_PREFILL, B=B, M=M, N=N, Hq=Hq, Hkv=Hkv, W=W, Di=Hq * 64)
    got, ref = _attn_case(shape, 2)
    assert_close(got, ref, "bf16", "attention bf16")


# positions offset by pos0 (a continued sequence; the angles reach 1e5 rad, where
# the kernels' double-precision reduction to revolutions matters) and a caller's
# softmax scale, through the standalone attention and the fused layer
@pytest.mark.parametrize("dtype,pos0,scale", [("f32", 37, 0.3), ("bf16", 5, 0.0),
                                              ("bf16", 100_000, 0.1)])
def test_attention_pos0_and_scale(dtype, pos0, scale):
    shape = with_(SWA_PREFILL, N=260, M=12, W=96, Hq=4, Hkv=2, Di=256, dtype=dtype)
    if dtype == "f32":
        shape = with_(shape, Hq=2, Hkv=1, Di=128, Dh=64)
    inp = prefill_inputs(shape, 7)
    t = up_inputs(inp, dtype)
    o = hm.swa_meta_attn(t["q"], t["k"], t["v"], shape.M, shape.W, shape.rope_base,
                         pos0=pos0, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], shape.M, shape.W, shape.rope_base,
                           pos0=pos0, scale=scale)
    assert_close(down(o), ref, dtype, "attention with pos0 / scale")


def test_mixer_prefill_bf16_pos0_and_scale():
    shape = with_(SWA_PREFILL, N=400, M=16, W=128)
    inp = prefill_inputs(shape, 8)
    r = hm.mixer_prefill(up_inputs(inp, "bf16"), shape.M, shape.W, pos0=4321, scale=0.11)
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill(inp, shape.M, shape.W, pos0=4321, scale=0.11)
    for k in ("ya", "ys", "out"):
        assert_close(down(r[k]), ref[k], "bf16", f"mixer {k} with pos0 / scale")


def test_attention_bf16_global_full_size_sampled_rows():
    # the global-attention workload at full size (B=4, T=8320), rows sampled
    # across tile boundaries, the meta prefix and the end
    shape = GLOBAL_PREFILL
    rows = sorted(set([0, 1, 63, 64, 127, 128, 129, 255, 1000, 4095, 4096, 6000, 8191, 8318,
                       8319] + list(np.random.default_rng(0).integers(0, shape.T, 17))))
    got, ref = _attn_case(shape, 3, rows=rows)
    assert_close(got, ref, "bf16", "attention global full size")


def test_global_layer_full_size():
    """The whole global-attention layer at full size (B=4, 128 + 8192 rows) in
    the launch configuration the benchmark times (the fused one-stream
    sequence): attention and fused output on rows sampled across query and
    key tiles, the end of the meta prefix and the last rows; the SSM branch on
    every row and its final conv and SSM states against a full sequential
    oracle scan."""
    shape = GLOBAL_PREFILL
    inp = prefill_inputs(shape, 4)
    t = up_inputs(inp, "bf16")
    plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
    plan.run()
    torch.cuda.synchronize()
    rows = np.array(sorted(set([0, 1, 63, 64, 127, 128, 129, 191, 192, 255, 256, 2047, 2048,
                                4160, 6000, 8191, 8255, 8256, 8318, 8319] +
                               list(np.random.default_rng(1).integers(0, shape.T, 12)))))
    ya_ref = oracle.attention(inp["q"], inp["k"], inp["v"], shape.M, shape.W, shape.rope_base,
                              rows=rows).reshape(shape.B, len(rows), shape.Di)
    assert_close(down(plan.ya)[:, rows], ya_ref, "bf16", "global layer attention rows")
    xc, cs_ref = oracle.causal_conv1d(inp["x"], inp["conv_w"], inp["conv_b"], None, True)
    ys_ref, h_ref = oracle.selective_scan(xc, inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                          inp["D"], inp["z"])
    assert_close(down(plan.ys), ys_ref, "bf16", "global layer ssm branch, every row")
    assert_close(down(plan.h), h_ref, "bf16", "global layer final ssm state")
    assert np.array_equal(down(plan.conv_state), cs_ref), "global layer final conv state"
    out_ref = oracle.branch_norm_mean(ya_ref, ys_ref[:, rows], inp["beta_a"], inp["beta_s"],
                                      shape.eps)
    assert_close(down(plan.out)[:, rows], out_ref, "bf16", "global layer out rows")


# ------------------------------------------------------------------ conv / scan / norm
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 5, 64, 200])
@pytest.mark.parametrize("with_state", [False, True])
def test_causal_conv1d(dtype, T, with_state):
    rng = np.random.default_rng(T)
    B, Di = 2, 96
    from workloads import bf16_round
    x = rng.standard_normal((B, T, Di)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    w = (rng.standard_normal((Di, 4)) / 2).astype(np.float32)
    b = (0.1 * rng.standard_normal(Di)).astype(np.float32)
    s0 = rng.standard_normal((B, Di, 3)).astype(np.float32) if with_state else None
    so = torch.empty((B, Di, 3), dtype=torch.float32, device="cuda")
    y = hm.causal_conv1d(up(x, dtype), up(w, "f32"), up(b, "f32"),
                         None if s0 is None else up(s0, "f32"), True, state_out=so)
    ref, ref_st = oracle.causal_conv1d(x, w, b, s0, True)
    assert_close(down(y), ref, dtype, "conv y")
    assert np.array_equal(down(so), ref_st), "conv state_out must be the exact inputs"


def _scan_inputs(shape, seed):
    inp = prefill_inputs(shape, seed)
    rng = np.random.default_rng(seed + 100)
    h0 = rng.standard_normal((shape.B, shape.Di, 16)).astype(np.float32)
    return inp, h0


@pytest.mark.parametrize("shape", [TINY, with_(TINY, dtype="bf16"),
                                   with_(SWA_PREFILL, N=2048, M=128),
                                   with_(SWA_PREFILL, B=3, N=777, M=11, Di=200, Hq=1, Dh=200)],
                         ids=["tiny-f32", "tiny-bf16", "swa-full", "ragged"])
@pytest.mark.parametrize("use_h0,use_dz", [(False, True), (True, True), (True, False)])
def test_selective_scan(shape, use_h0, use_dz):
    inp, h0 = _scan_inputs(shape, 5)
    dt = shape.dtype
    t = up_inputs(inp, dt)
    h_out = torch.empty((shape.B, shape.Di, 16), dtype=torch.float32, device="cuda")
    y = hm.selective_scan(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"],
                          t["D"] if use_dz else None, t["z"] if use_dz else None,
                          up(h0, "f32") if use_h0 else None, h_out=h_out)
    ref, ref_h = oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                       inp["D"] if use_dz else None, inp["z"] if use_dz else None,
                                       h0 if use_h0 else None)
    assert_close(down(y), ref, dt, "scan y")
    assert_close(down(h_out), ref_h, dt, "scan h_out")


@pytest.mark.parametrize("shape", [TINY, with_(SWA_PREFILL, N=2048, M=128),
                                   with_(SWA_PREFILL, B=2, N=500, M=7, Di=320, Hq=5),
                                   with_(SWA_PREFILL, B=4, N=1920, M=128)],
                         ids=["tiny-f32", "swa-full", "ragged", "long-two-launch"])
@pytest.mark.parametrize("use_state", [False, True])
def test_conv_selective_scan(shape, use_state):
    """The last shape (4 x 2048 rows, 4200 aggregate waves) takes the two-launch
    form whose final pass composes its own incoming states; the others the
    aggregate, carry and final launches."""
    inp, h0 = _scan_inputs(shape, 6)
    rng = np.random.default_rng(7)
    cs0 = rng.standard_normal((shape.B, shape.Di, 3)).astype(np.float32) if use_state else None
    dt = shape.dtype
    t = up_inputs(inp, dt)
    h_out = torch.empty((shape.B, shape.Di, 16), dtype=torch.float32, device="cuda")
    cs_out = torch.empty((shape.B, shape.Di, 3), dtype=torch.float32, device="cuda")
    y = hm.conv_selective_scan(t["x"], t["conv_w"], t["conv_b"], t["delta"], t["A"], t["Bm"],
                               t["Cm"], t["D"], t["z"],
                               conv_state_in=None if cs0 is None else up(cs0, "f32"),
                               conv_state_out=cs_out, h0=up(h0, "f32") if use_state else None,
                               h_out=h_out)
    xc, ref_cs = oracle.causal_conv1d(inp["x"], inp["conv_w"], inp["conv_b"], cs0, True)
    ref, ref_h = oracle.selective_scan(xc, inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["D"],
                                       inp["z"], h0 if use_state else None)
    assert_close(down(y), ref, dt, "conv+scan y")
    assert_close(down(h_out), ref_h, dt, "conv+scan h_out")
    assert np.array_equal(down(cs_out), ref_cs)


@pytest.mark.parametrize("dtype,width,rows", [("f32", 32, 64), ("bf16", 1600, 2176),
                                              ("bf16", 1600, 3), ("f32", 37, 5),
                                              ("bf16", 200, 9), ("bf16", 2400, 7),
                                              ("f32", 2048, 6),
                                              # packed bf16 rows: the widest (2048), one
                                              # 8-element chunk, and 65 chunks (lane 0 two)
                                              ("bf16", 2048, 5), ("bf16", 8, 4),
                                              ("bf16", 520, 33)])
def test_branch_norm_mean(dtype, width, rows):
    rng = np.random.default_rng(width)
    from workloads import bf16_round
    ya = (0.3 * rng.standard_normal((rows, width))).astype(np.float32)
    ys = (30 * rng.standard_normal((rows, width))).astype(np.float32)
    if dtype == "bf16":
        ya, ys = bf16_round(ya), bf16_round(ys)
    ba = (1 + 0.1 * rng.standard_normal(width)).astype(np.float32)
    bs = (1 + 0.1 * rng.standard_normal(width)).astype(np.float32)
    out = hm.branch_norm_mean(up(ya, dtype), up(ys, dtype), up(ba, "f32"), up(bs, "f32"), 1e-6)
    ref = oracle.branch_norm_mean(ya, ys, ba, bs, 1e-6)
    assert_close(down(out), ref, dtype, "norm-mean")


# ------------------------------------------------------------------ whole layer
@pytest.mark.parametrize("shape", [TINY, SWA_PREFILL], ids=["tiny-f32", "swa-prefill-full"])
def test_mixer_prefill(shape):
    inp = prefill_inputs(shape, 0)
    t = up_inputs(inp, shape.dtype)
    r = hm.mixer_prefill(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill(inp, shape.M, shape.W, shape.rope_base, shape.eps)
    for k in ("ya", "ys", "out", "ssm_state"):
        assert_close(down(r[k]), ref[k], shape.dtype, f"mixer {k}")
    assert np.array_equal(down(r["conv_state"]), ref["conv_state"])


# bf16 layers on one stream take the fused launch sequence (pre-pass | chunk
# aggregates, attention | final pass with its own carry, norm): short sequences with a
# single scan chunk, ragged lengths, several sequences, global attention
@pytest.mark.parametrize("B,M,N,W,Hq,Hkv", [(1, 4, 20, 16, 5, 5), (1, 5, 77, 32, 4, 2),
                                            (2, 16, 300, 64, 10, 5), (3, 0, 129, 0, 5, 1),
                                            (1, 128, 1000, 1024, 25, 5)])
def test_mixer_prefill_bf16_fused_shapes(B, M, N, W, Hq, Hkv):
    shape = with_(SWA_PREFILL, B=B, M=M, N=N, W=W, Hq=Hq, Hkv=Hkv, Di=Hq * 64)
    inp = prefill_inputs(shape, 21 + N)
    t = up_inputs(inp, "bf16")
    r = hm.mixer_prefill(t, shape.M, shape.W)
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill(inp, shape.M, shape.W)
    for k in ("ya", "ys", "out", "ssm_state"):
        assert_close(down(r[k]), ref[k], "bf16", f"mixer {k}")
    assert np.array_equal(down(r["conv_state"]), ref["conv_state"])


def test_mixer_prefill_kv_reuse_one_stream():
    shape = with_(SWA_PREFILL, N=400, M=32, W=128)
    prod, cons = prefill_inputs(shape, 14), prefill_inputs(shape, 15)
    tp, tc = up_inputs(prod, "bf16"), up_inputs(cons, "bf16")
    del tc["k"], tc["v"]
    tc["Hkv"] = shape.Hkv
    p1 = hm.PrefillPlan(tp, shape.M, shape.W)
    p2 = hm.PrefillPlan(tc, shape.M, shape.W, kv=p1.kv, kv_reuse=True)
    p1.run()
    p2.run()
    torch.cuda.synchronize()
    mixed = dict(cons)
    mixed["k"], mixed["v"] = prod["k"], prod["v"]
    for plan, src in ((p1, prod), (p2, mixed)):
        ref = oracle.mixer_prefill(src, shape.M, shape.W)
        for k, got in (("ya", plan.ya), ("ys", plan.ys), ("out", plan.out)):
            assert_close(down(got), ref[k], "bf16", k)


# ------------------------------------------------------------------ timing events
def test_mixer_prefill_events_leave_results_unchanged():
    """The optional events are recorded between the fused launches and change
    nothing else: outputs bit-identical to a run without them, the recorded
    intervals non-negative, and a NULL entry skipped."""
    shape = with_(SWA_PREFILL, N=600, M=32, W=128)
    t = up_inputs(prefill_inputs(shape, 31), "bf16")
    plan = hm.PrefillPlan(t, shape.M, shape.W)
    plan.run()
    torch.cuda.synchronize()
    base = {k: getattr(plan, k).clone() for k in ("ya", "ys", "out", "h")}
    for skip in (None, 2):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        use = [None if i == skip else e for i, e in enumerate(evs)]
        plan.run(events=use)
        torch.cuda.synchronize()
        for k, ref in base.items():
            assert torch.equal(getattr(plan, k), ref), k
        live = [e for e in use if e is not None]
        gaps = [a.elapsed_time(b) for a, b in zip(live, live[1:])]
        assert all(g >= 0 for g in gaps), gaps
        assert live[0].elapsed_time(live[-1]) > 0


# ------------------------------------------------------------------ prepared K/V, two streams
def test_prepared_kv_shared_between_layers():
    shape = with_(SWA_PREFILL, N=500, M=16, W=128)
    prod, cons = prefill_inputs(shape, 10), prefill_inputs(shape, 11)
    tp, tc = up_inputs(prod, "bf16"), up_inputs(cons, "bf16")
    kv = hm.attn_kv_prepare(tp["k"], tp["v"])
    o = hm.attn_with_kv(tc["q"], kv, shape.Hkv, shape.M, shape.W)
    ref = oracle.attention(cons["q"], prod["k"], prod["v"], shape.M, shape.W)
    assert_close(down(o), ref, "bf16", "consumer attention over producer K/V")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixer_prefill_two_streams_and_kv_reuse(dtype):
    shape = with_(SWA_PREFILL, N=700, M=64, W=256, dtype=dtype) if dtype == "bf16" else \
        with_(TINY, N=200, Hq=4, Hkv=2, Di=64)
    prod, cons = prefill_inputs(shape, 12), prefill_inputs(shape, 13)
    tp, tc = up_inputs(prod, dtype), up_inputs(cons, dtype)
    del tc["k"], tc["v"]
    tc["Hkv"] = shape.Hkv
    s2 = torch.cuda.Stream()
    p1 = hm.PrefillPlan(tp, shape.M, shape.W, stream2=s2)
    p2 = hm.PrefillPlan(tc, shape.M, shape.W, kv=p1.kv, kv_reuse=True, stream2=s2)
    for _ in range(2):       # a second run reuses the same buffers and events
        p1.run()
        p2.run()
    torch.cuda.synchronize()
    mixed = dict(cons)
    mixed["k"], mixed["v"] = prod["k"], prod["v"]
    for plan, src in ((p1, prod), (p2, mixed)):
        ref = oracle.mixer_prefill(src, shape.M, shape.W)
        for k, got in (("ya", plan.ya), ("ys", plan.ys), ("out", plan.out), ("ssm_state", plan.h)):
            assert_close(down(got), ref[k], dtype, f"{k}")


# ------------------------------------------------------------------ cached meta tokens
def _cached_meta_run(shape, seed, cache=None):
    """Prefill of the real tokens with the meta rows cached, against the
    oracle's cached-meta prefill (itself pinned against the full prefill)."""
    full, tokens, meta = cached_meta_inputs(shape, seed)
    if cache is None:
        cache = oracle.meta_cache(meta)
        # the GPU takes the states in float32
        cache["ssm_state"] = cache["ssm_state"].astype(np.float32).astype(np.float64)
    B = shape.B
    t = up_inputs(tokens, "bf16")
    mk = up(meta["k"], "bf16")
    mv = up(meta["v"], "bf16")
    cs = up(np.broadcast_to(cache["conv_state"], (B,) + cache["conv_state"].shape).copy(), "f32")
    h0 = up(np.broadcast_to(cache["ssm_state"], (B,) + cache["ssm_state"].shape).copy(), "f32")
    plan = hm.PrefillPlan(t, shape.M, shape.W, meta={"k": mk, "v": mv}, conv_state_in=cs, h0=h0)
    plan.run()
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill_cached_meta(tokens, cache, shape.M, shape.W)
    return plan, ref


@pytest.mark.parametrize("B,M,N,W,Hq,Hkv", [(1, 128, 2048, 1024, 25, 5), (2, 5, 77, 32, 4, 2),
                                            (3, 16, 300, 0, 5, 1), (1, 4, 20, 16, 5, 5),
                                            (2, 130, 40, 64, 10, 5), (1, 64, 1, 32, 2, 1)])
def test_mixer_prefill_bf16_cached_meta(B, M, N, W, Hq, Hkv):
    """Only the real tokens computed, the meta rows' K/V and the SSM-branch
    states after them taken from a cache: short and ragged token counts, meta
    counts off the tile grid, several sequences, global attention."""
    shape = with_(SWA_PREFILL, B=B, M=M, N=N, W=W, Hq=Hq, Hkv=Hkv, Di=Hq * 64)
    plan, ref = _cached_meta_run(shape, 40 + N)
    for k, got in (("ya", plan.ya), ("ys", plan.ys), ("out", plan.out), ("ssm_state", plan.h)):
        assert_close(down(got), ref[k], "bf16", f"cached meta {k}")
    assert np.array_equal(down(plan.conv_state), ref["conv_state"])


def test_mixer_prefill_cached_meta_states_from_the_library():
    """The documented workflow: the meta rows alone through hm_mixer_prefill
    (one sequence) give the states; the cached prefill of the tokens then
    equals the last rows of the full prefill over [meta; tokens]."""
    shape = with_(SWA_PREFILL, B=2, M=32, N=200, W=64, Hq=5, Hkv=1, Di=320)
    full, tokens, meta = cached_meta_inputs(shape, 9)
    mshape = with_(shape, B=1, N=0)
    mt = up_inputs({k: (v[None] if k in ("q", "k", "v", "x", "delta", "Bm", "Cm", "z") else v)
                    for k, v in meta.items()}, "bf16")
    mplan = hm.PrefillPlan(mt, mshape.M, mshape.W)
    mplan.run()
    t = up_inputs(tokens, "bf16")
    cs = mplan.conv_state.expand(shape.B, -1, -1).contiguous()
    h0 = mplan.h.expand(shape.B, -1, -1).contiguous()
    plan = hm.PrefillPlan(t, shape.M, shape.W, meta={"k": mt["k"][0], "v": mt["v"][0]},
                          conv_state_in=cs, h0=h0)
    plan.run()
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill(full, shape.M, shape.W)
    for k, got in (("ya", plan.ya), ("ys", plan.ys), ("out", plan.out), ("ssm_state", plan.h)):
        ref_k = ref[k][:, shape.M:] if k != "ssm_state" else ref[k]
        assert_close(down(got), ref_k, "bf16", f"cached meta via the library, {k}")
