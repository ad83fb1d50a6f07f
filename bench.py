#!/usr/bin/env python3
"""Benchmark of the Hymba hybrid-head mixer core on one MI355X.

A step is one prefill pass of one mixer layer (RoPE, the meta + sliding-window
GQA attention, the causal conv + selective scan branch, the branch norm and
average; all kernels in order on one stream) over the sliding-window
workload: batch 1, 128 meta + 2048 tokens, 25 query heads x 64, 5 KV heads,
window 1024, SSM width 1600 x 16 states, bf16 inputs with float32
accumulation, synthetic seeded inputs resident in HBM.
`value` is prefill tokens/s per layer (B * (M + N) rows / step time).

Also reported on the same JSON line:
  roofline      the attention kernel (the dominant one) timed on its own with
                HIP events on its stream: algorithmic FLOPs / time vs the bf16
                MFMA peak;
  decode        one token for 64 sequences through an adjacent pair of layers
                that share a 128 + 1024-row KV cache: steps/s and HBM fraction,
                with the Infinity Cache flushed before each step (and warm);
  global_prefill, stack
                the global-attention layer (batch 4, 128 + 8192 tokens) and the
                32-layer stack (batch 2, 128 + 16384 tokens, layers 0/15/31
                global, adjacent sliding-window layers sharing prepared K/V);
  ragged_decode the decode pair with one n_prev per sequence (warm);
  projections   the in- and out-projections around the layer (bf16 MFMA GEMM);
  block         one whole Hymba block (RMS norm, in-projection, step-size/B/C
                projection, the mixer, out-projection with the skip connection,
                RMS norm, FFN 1600 -> 5504 -> 1600 with the skip connection) over
                the same rows at the model card's widths;
  block_stack   32 whole blocks chained over one hidden-state tensor at the
                stack's size (batch 2, 128 + 16384 tokens; KV shared as above);
  cached_meta   the same layer with the meta tokens' K/V and SSM states taken
                from a cache: only the 2048 real-token rows are computed
                (real tokens/s, beside the full layer's real tokens/s);
  layer_step_us single-call times of the step (median, p10, p90) after the timed
                region, and (sclk_mhz) the shader clock the driver reports while
                those calls run;
  ssm_branch    the conv + scan branch on its own against HBM and against the
                non-packed fp32 VALU rate (single-pass VALU work per
                token-channel);
  cpu_baseline  the float64 CPU oracle on one whole layer of the step's workload.
HBM traffic (`traffic`) of the attention kernel, the SSM branch, the decode pair
and the block stack's in-projection GEMM (block_stack.roofline, the block's
dominant kernel timed on its own) comes from the committed rocprofv3 counter
summaries in profiles/ (null
once the kernel sources differ from those the counters were taken with);
`--counters` is the run those summaries are taken over.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
                       [--no-cpu-baseline] [--counters]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
COPY_BYTES = 256 << 20      # calibration copy for the HBM byte counters
# sources of the kernels whose HBM counters profiles/ holds
ATTN_SOURCES = ("hybrid_head_lm_amd/csrc/attn_dev.h", "hybrid_head_lm_amd/csrc/attn.hip",
                "hybrid_head_lm_amd/csrc/hm_common.h")
SSM_SOURCES = ("hybrid_head_lm_amd/csrc/ssm_dev.h", "hybrid_head_lm_amd/csrc/ssm.hip",
               "hybrid_head_lm_amd/csrc/hm_common.h")
STEP_SOURCES = ("hybrid_head_lm_amd/csrc/step.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
LINEAR_SOURCES = ("hybrid_head_lm_amd/csrc/linear_w4.hip", "hybrid_head_lm_amd/csrc/linear_dev.h",
                  "hybrid_head_lm_amd/csrc/linear.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
PEAK_VALU_LANE_OPS = 256 * 64 * 2.4e9   # non-packed fp32 VALU: 64 lanes/clk/CU
# single-pass VALU work of the SSM branch per token-channel: per state the decay
# product, exp, h product, input term, output term (4 VALU + 1 transcendental);
# per token-channel the conv (4), SiLU of the conv (3 + 2), delta*x (1), D*x (1),
# the gate SiLU(z) (3 + 2) and the gate product (1)
SCAN_VALU_PER_TC = 16 * 4 + 4 + 3 + 1 + 1 + 3 + 1
SCAN_TRANS_PER_TC = 16 + 2 + 2


def attn_flops(shape) -> float:
    """4 * Dh * Hq * B * (visible (query, key) pairs per head) — QK^T and PV only."""
    import numpy as np
    i = np.arange(shape.T, dtype=np.int64)
    vis = np.minimum(i + 1, shape.M + shape.W) if shape.W > 0 else i + 1
    return 4.0 * shape.Dh * shape.Hq * shape.B * float(vis.sum())


def scan_bytes(shape) -> float:
    """Compulsory HBM bytes of the SSM branch: read x, delta, z, write y (2 B each
    per token-channel), read B and C (2 B per token-state), A, D, conv params once."""
    tc = shape.B * shape.T * shape.Di
    return 8.0 * tc + 4.0 * shape.B * shape.T * shape.Ns + 4.0 * shape.Di * (shape.Ns + 1 + 5)


def decode_bytes(shape, n_prev_seq=None) -> float:
    """Compulsory HBM bytes of one decode token through a producer + consumer
    layer: both read the visible cache rows (K and V), each reads and writes its
    SSM and conv states, reads q, x, delta, z, B, C and writes out; the producer
    reads k_new, v_new and writes them into the cache.  n_prev_seq: one n_prev
    per sequence (ragged batch)."""
    B, Hkv, Dh, Di, Ns = shape.B, shape.Hkv, shape.Dh, shape.Di, shape.Ns
    nps = [shape.n_prev] * B if n_prev_seq is None else list(n_prev_seq)
    rows = sum(shape.M + (min(n + 1, shape.W) if shape.W > 0 else n + 1) for n in nps)
    per_layer = (rows * Hkv * Dh * 2 * 2               # K and V rows
                 + B * Di * Ns * 4 * 2                 # SSM state read + write
                 + B * Di * 3 * 4 * 2                  # conv state read + write
                 + B * shape.Hq * Dh * 2               # q
                 + B * Di * 2 * 4                      # x, delta, z, out
                 + B * Ns * 2 * 2)                     # B, C
    producer = B * Hkv * Dh * 2 * 2 * 2                # k_new, v_new read + written
    return 2.0 * per_layer + producer


def _sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_srcs, summary: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes (per launch, or per the unit `key` names) from a committed
    rocprofv3 counter summary, or None when there is none or the kernel sources
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != _sources_hash(kernel_srcs):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def timed(fn, steps: int, warmup: int, stream=None):
    """Mean milliseconds per call over `steps` calls, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = stream or torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_percentiles(fn, steps: int, while_busy=None):
    """Median, p10 and p90 of single-call times (microseconds), one HIP event
    pair around each call, after the timed region (a distribution, not the
    headline figure).  `while_busy` runs on the host once every call is queued,
    while the GPU is still working through them."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    if while_busy is not None:
        while_busy()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    pick = lambda q: us[min(len(us) - 1, int(q * (len(us) - 1) + 0.5))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "calls": len(us)}


def gpu_sclk_mhz():
    """(current, highest level) shader clock in MHz from the driver's sysfs
    table (the current one is the line marked *), or (None, None)."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            cur, top = None, None
            for line in open(f):
                mhz = float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
                top = mhz if top is None else max(top, mhz)
                if line.rstrip().endswith("*"):
                    cur = mhz
            return cur, top
        except (OSError, ValueError, IndexError):
            continue
    return None, None


def sample_sclk(samples: list, n: int = 12, gap_s: float = 0.001):
    """Read the current shader clock n times, gap_s apart (while the GPU works)."""
    for _ in range(n):
        samples.append(gpu_sclk_mhz())
        time.sleep(gap_s)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(shape, inp, min_seconds: float = 10.0):
    """The oracle (float64 NumPy) on whole prefill layers of the workload,
    repeated until at least `min_seconds` of CPU work have been timed."""
    import oracle
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((d.get("num_threads") or 1) for d in info) if info else 1
    except Exception:
        pass
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.mixer_prefill(inp, shape.M, shape.W, shape.rope_base, shape.eps)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": n * shape.B * shape.T / dt, "unit": "tokens/s", "cores": threads or 1,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} whole prefill layers of {shape.name} (float64 NumPy, same "
                      f"inputs each time), {dt:.1f} s"}


def run_prefill(shape, hm, t, steps, warmup, two_streams):
    import torch
    s2 = torch.cuda.Stream() if two_streams else None
    plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps,
                          want_states=False, stream2=s2)
    ms = timed(plan.run, steps, warmup)
    return plan, ms


def run_stack(shape, hm, steps, warmup):
    """32 layers; sliding-window pairs share the producer's prepared K/V."""
    import torch
    from workloads import prefill_inputs_torch, stack_layer_roles
    roles = stack_layer_roles(shape)
    layers = []
    for layer, (_, src) in enumerate(roles):
        t = prefill_inputs_torch(shape, 0, layer, torch.device("cuda"))
        if src != layer:
            del t["k"], t["v"]
        layers.append(t)
    # one stream: every layer takes the fused three-launch sequence (measured
    # 26.2 ms against 28.0 ms with the SSM branch on a second stream)
    stack = hm.StackPlan(layers, roles, shape.M, shape.rope_base, shape.eps)
    ms = timed(stack.run, steps, warmup)
    return ms, len(roles)


def block_matmul_flops(shape, producer: bool = True) -> float:
    """Dense products of one block: in-projection, the step-size/B/C
    projection, out-projection and the two FFN matrices (2 flops per MAC)."""
    from workloads import block_weight_rows
    R = shape.B * shape.T
    macs = (shape.d_model * block_weight_rows(shape, producer)
            + shape.Di * (shape.Di + 2 * shape.Ns) + shape.Di * shape.d_model
            + 2 * shape.d_model * shape.d_ffn)
    return 2.0 * R * macs


def block_in_proj_operands(shape):
    """The in-projection of a producer block at ``shape``: x [B*T, d] and the weight with
    rows Q, K, V, x, z (device generator), and the segment widths."""
    import torch
    from workloads import block_inputs_torch
    dev = torch.device("cuda")
    t = block_inputs_torch(shape, 0, 0, True, dev, hidden=True)
    x = t["hidden"].reshape(-1, shape.d_model).contiguous()
    kvw = shape.Hkv * shape.Dh
    return x, t["w_in"], [shape.Hq * shape.Dh, kvw, kvw, shape.Di, shape.Di]


def run_blocks(shape, hm, n_layers, steps, warmup):
    """Whole blocks (norm, projections, mixer, norm, FFN) chained over one
    hidden-state tensor; weights from the device generator.  Returns ms per
    pass and the pass's dense-product and attention flops."""
    import torch
    from workloads import block_inputs_torch, stack_layer_roles, with_
    dev = torch.device("cuda")
    roles = stack_layer_roles(with_(shape, layers=n_layers)) if n_layers > 1 else [(shape.W, 0)]
    layers = [block_inputs_torch(shape, 0, l, src == l, dev, hidden=(l == 0))
              for l, (_, src) in enumerate(roles)]
    hidden = layers[0].pop("hidden")
    stack = hm.BlockStack(layers, roles, hidden, shape.Hq, shape.Hkv, shape.M, shape.rope_base,
                          shape.eps)
    ms = timed(stack.run, steps, warmup)
    fl_mm = sum(block_matmul_flops(shape, src == l) for l, (_, src) in enumerate(roles))
    fl_at = sum(attn_flops(with_(shape, W=w)) for w, _ in roles)
    del stack, layers, hidden
    return ms, len(roles), fl_mm, fl_at


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="skip the global-prefill and stack lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="only a 256 MiB device copy (calibration) and the kernels whose HBM "
                         "counters profiles/ holds, for rocprofv3 --pmc runs; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the mixer core runs on a single MI355X here "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import hybrid_head_lm_amd as hm
    from workloads import (BLOCK_STACK, BLOCK_SWA, DECODE_PAIR, GLOBAL_PREFILL, STACK,
                           SWA_PREFILL, decode_inputs, prefill_inputs, to_device)

    torch.cuda.set_device(0)
    shape = SWA_PREFILL
    inp = prefill_inputs(shape, 0)
    t = to_device(inp, shape.dtype)

    if args.counters:
        plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
        plan.run()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            hm.attn_with_kv(t["q"], plan.kv, shape.Hkv, shape.M, shape.W, shape.rope_base,
                            out=plan.ya)
        for _ in range(3):
            hm.conv_selective_scan(t["x"], t["conv_w"], t["conv_b"], t["delta"], t["A"],
                                   t["Bm"], t["Cm"], t["D"], t["z"], out=plan.ys)
        for _ in range(3):
            plan.run()
        dshape = DECODE_PAIR
        d = to_device(decode_inputs(dshape, 0), dshape.dtype)
        pa = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W)
        pb = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W)
        for _ in range(3):
            pa.run()
            pb.run()
        del pa, pb, d
        x, w, segs = block_in_proj_operands(BLOCK_STACK)
        outs = [torch.empty((x.shape[0], c), dtype=torch.bfloat16, device="cuda") for c in segs]
        for _ in range(3):
            hm.linear(x, w, seg_cols=segs, outs=outs)
        torch.cuda.synchronize()
        print("counters run done: 3 copies of", COPY_BYTES, "bytes, then 3 each of the "
              "attention launch, the SSM branch, the fused layer, the decode pair and the "
              "block-stack in-projection")
        return

    # the step: one mixer layer (both branches on one stream, kernels in order)
    plan, ms = run_prefill(shape, hm, t, args.steps, args.warmup, two_streams=False)
    sclk = []
    layer_dist = step_percentiles(plan.run, max(200, args.steps),
                                  while_busy=lambda: sample_sclk(sclk))
    cur = [c for c, _ in sclk if c is not None]
    sclk = {"max_sampled": max(cur) if cur else None,
            "highest_level": sclk[0][1] if sclk else None,
            "note": "the driver's current-clock line (S:), read 12 times 1 ms apart while "
                    "the layer calls run; it reads far below the highest level and below what "
                    "the measured MFMA rates need, so it is an average that includes idle "
                    "time, not the clock during the kernels"}
    _, ms_two = run_prefill(shape, hm, t, args.steps, args.warmup, two_streams=True)
    tokens = shape.B * shape.T

    # the same layer with the meta tokens cached: only the N real-token rows are
    # computed, from the meta rows' K/V and the SSM-branch states after them
    from workloads import cached_meta_inputs
    _, ctok, cmeta = cached_meta_inputs(shape, 0)
    ct = to_device(ctok, shape.dtype)
    cmk = to_device({"k": cmeta["k"], "v": cmeta["v"]}, shape.dtype)
    cst = torch.zeros((shape.B, shape.Di, shape.K - 1), dtype=torch.float32, device="cuda")
    ch0 = torch.zeros((shape.B, shape.Di, shape.Ns), dtype=torch.float32, device="cuda")
    cplan = hm.PrefillPlan(ct, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps,
                           want_states=False, meta={"k": cmk["k"], "v": cmk["v"]},
                           conv_state_in=cst, h0=ch0)
    ms_cached = timed(cplan.run, args.steps, args.warmup)
    del cplan, ct, cmk

    # the projections around the layer: in-projection of the 2176 rows from width
    # 1600 into Q, K, V, x, z (5440 columns) and the out-projection (1600 -> 1600)
    gen = torch.Generator(device="cuda").manual_seed(3)
    d_model = shape.Hq * shape.Dh
    segs = [shape.Hq * shape.Dh, shape.Hkv * shape.Dh, shape.Hkv * shape.Dh, shape.Di, shape.Di]
    px = torch.randn(shape.B * shape.T, d_model, device="cuda", generator=gen).bfloat16()
    pw_in = (torch.randn(sum(segs), d_model, device="cuda", generator=gen)
             / d_model ** 0.5).bfloat16()
    pw_out = (torch.randn(d_model, shape.Di, device="cuda", generator=gen)
              / shape.Di ** 0.5).bfloat16()
    pouts = [torch.empty(shape.B * shape.T, c, dtype=torch.bfloat16, device="cuda") for c in segs]
    py = torch.empty(shape.B * shape.T, d_model, dtype=torch.bfloat16, device="cuda")
    ms_in = timed(lambda: hm.linear(px, pw_in, seg_cols=segs, outs=pouts), args.steps, args.warmup)
    ms_out = timed(lambda: hm.linear(pouts[3], pw_out, outs=[py]), args.steps, args.warmup)
    fl_in = 2.0 * shape.B * shape.T * sum(segs) * d_model
    fl_out = 2.0 * shape.B * shape.T * d_model * shape.Di
    del px, pw_in, pw_out, pouts, py

    # dominant kernel on its own: attention over the prepared K/V
    ms_attn = timed(lambda: hm.attn_with_kv(t["q"], plan.kv, shape.Hkv, shape.M, shape.W,
                                            shape.rope_base, out=plan.ya),
                    args.steps, args.warmup)
    fl = attn_flops(shape)
    achieved = fl / (ms_attn * 1e-3) / 1e12
    traffic = traffic_from_profile(ATTN_SOURCES, "attn_fwd_bf16.swa-prefill-b1-t2176.pmc.txt")

    # SSM branch and fusion on their own (context for the breakdown)
    tc_ssm = shape.B * shape.T * shape.Di
    ms_ssm = timed(lambda: hm.conv_selective_scan(t["x"], t["conv_w"], t["conv_b"], t["delta"],
                                                  t["A"], t["Bm"], t["Cm"], t["D"], t["z"],
                                                  out=plan.ys), args.steps, args.warmup)
    ms_norm = timed(lambda: hm.branch_norm_mean(plan.ya, plan.ys, t["beta_a"], t["beta_s"],
                                                shape.eps, out=plan.out), args.steps, args.warmup)

    # decode: one token through the producer / consumer pair
    dshape = DECODE_PAIR
    d = to_device(decode_inputs(dshape, 0), dshape.dtype)
    pa = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W,
                     rope_base=dshape.rope_base, eps=dshape.eps)
    pb = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W,
                     rope_base=dshape.rope_base, eps=dshape.eps)

    def decode_step():
        pa.run()
        pb.run()
    ms_dec = timed(decode_step, args.steps, args.warmup)
    dbytes = decode_bytes(dshape)
    # cold: before every step a 512 MB write evicts the pair's cache and states
    # from the 256 MB Infinity Cache, as the other layers of a model would, and a
    # 1 GB read then leaves the cache holding clean lines (the other layers
    # mostly read weights and caches), so the step does not pay for writing back
    # the flush's dirty lines
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush_rd = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cold = []
    for i in range(args.warmup + args.steps):
        flush.fill_(i & 0xFF)
        flush_rd.max()
        e0.record()
        decode_step()
        e1.record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            cold.append(e0.elapsed_time(e1))
    ms_dec_cold = sum(cold) / len(cold)
    del flush, flush_rd

    # ragged decode: the same pair with one n_prev per sequence, uniform over
    # 0 .. 2047 (seeded), back to back
    import numpy as np
    nps = np.random.default_rng(5).integers(0, 2048, size=dshape.B).astype(np.int32)
    npt = torch.from_numpy(nps).cuda()
    ra_plan = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], int(nps.max()), dshape.M, dshape.W,
                          rope_base=dshape.rope_base, eps=dshape.eps, n_prev_seq=npt)
    rb_plan = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], int(nps.max()), dshape.M, dshape.W,
                          rope_base=dshape.rope_base, eps=dshape.eps, n_prev_seq=npt)

    def ragged_step():
        ra_plan.run()
        rb_plan.run()
    ms_rag = timed(ragged_step, args.steps, args.warmup)
    rag_bytes = decode_bytes(dshape, nps)
    del ra_plan, rb_plan

    result = {
        "metric": "hybrid-mixer prefill tokens/s per layer + decode steps/s; % MFMA/HBM roofline",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": shape.name, "batch": shape.B, "meta_tokens": shape.M,
                   "tokens": shape.N, "rows": shape.T, "q_heads": shape.Hq,
                   "kv_heads": shape.Hkv, "head_dim": shape.Dh, "window": shape.W,
                   "ssm_width": shape.Di, "ssm_states": shape.Ns, "conv": shape.K,
                   "branches": "attention then SSM on one stream"},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "algorithmic_flop_per_launch": fl, "ms_per_launch": ms_attn},
        "cached_meta": {"workload": shape.name + " with the 128 meta rows cached",
                        "real_tokens_per_s": shape.B * shape.N / (ms_cached * 1e-3),
                        "ms_per_layer": ms_cached,
                        "full_layer_real_tokens_per_s": shape.B * shape.N / (ms * 1e-3)},
        "projections": {
            "workload": shape.name + " in-projection 1600 -> Q, K, V, x, z (5440) and "
                                     "out-projection 1600 -> 1600, bf16",
            "in_proj": {"ms": ms_in, "achieved": fl_in / (ms_in * 1e-3) / 1e12,
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": fl_in / (ms_in * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
            "out_proj": {"ms": ms_out, "achieved": fl_out / (ms_out * 1e-3) / 1e12,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": fl_out / (ms_out * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}},
        "layer_step_us": layer_dist,
        "sclk_mhz": sclk,
        "breakdown_ms": {"layer_one_stream": ms, "layer_two_streams": ms_two,
                         "attention_kernel": ms_attn, "ssm_branch": ms_ssm,
                         "norm_mean": ms_norm},
        "ssm_branch": {"bound": "hbm", "achieved": scan_bytes(shape) / (ms_ssm * 1e-3) / 1e9,
                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": scan_bytes(shape) / (ms_ssm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                       "traffic": traffic_from_profile(
                           SSM_SOURCES, "ssm-branch.swa-prefill-b1-t2176.pmc.txt",
                           "hbm_bytes_per_call"),
                       "alu": {"bound": "alu", "unit": "lane-op/s",
                               "valu_per_token_channel": SCAN_VALU_PER_TC,
                               "transcendental_per_token_channel": SCAN_TRANS_PER_TC,
                               "achieved": tc_ssm * (SCAN_VALU_PER_TC + SCAN_TRANS_PER_TC)
                                           / (ms_ssm * 1e-3),
                               "peak": PEAK_VALU_LANE_OPS,
                               "frac": tc_ssm * (SCAN_VALU_PER_TC + SCAN_TRANS_PER_TC)
                                       / (ms_ssm * 1e-3) / PEAK_VALU_LANE_OPS}},
        "decode": {"workload": dshape.name, "steps_per_s": 1e3 / ms_dec_cold,
                   "tokens_per_s": dshape.B * 1e3 / ms_dec_cold, "ms_per_step": ms_dec_cold,
                   "cache": "cold (Infinity Cache flushed before every step: 512 MB "
                            "written, then 1 GB read)",
                   "roofline": {"bound": "hbm",
                                "achieved": dbytes / (ms_dec_cold * 1e-3) / 1e9,
                                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": dbytes / (ms_dec_cold * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                "algorithmic_bytes_per_step": dbytes,
                                "traffic": traffic_from_profile(
                                    STEP_SOURCES, "step-pair.decode-pair-b64-cache1152.pmc.txt",
                                    "hbm_bytes_per_step")},
                   "warm": {"steps_per_s": 1e3 / ms_dec, "ms_per_step": ms_dec,
                            "hbm_frac": dbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                            "note": "back-to-back steps; the 222 MB of the pair stay in the "
                                    "256 MB Infinity Cache"}},
        "ragged_decode": {"workload": dshape.name + " with n_prev per sequence uniform "
                                                    "over 0..2047 (seeded)",
                          "steps_per_s": 1e3 / ms_rag, "ms_per_step": ms_rag,
                          "hbm_frac": rag_bytes / (ms_rag * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                          "algorithmic_bytes_per_step": rag_bytes,
                          "cache": "warm (back-to-back steps)"},
    }
    del pa, pb, d

    # one whole block at the model card's widths over the same rows
    bshape = BLOCK_SWA
    bms, _, bfl_mm, bfl_at = run_blocks(bshape, hm, 1, args.steps, args.warmup)
    result["block"] = {
        "workload": bshape.name + " (width 1600, FFN 5504; norm, projections, mixer, norm, FFN)",
        "tokens_per_s": bshape.B * bshape.T / (bms * 1e-3), "ms_per_block": bms,
        "mixer_ms": ms, "matmul_tflop": bfl_mm / 1e12,
        "tflops": (bfl_mm + bfl_at) / (bms * 1e-3) / 1e12,
        "frac_mfma": (bfl_mm + bfl_at) / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    torch.cuda.empty_cache()

    if not args.quick:
        gshape = GLOBAL_PREFILL
        gt = to_device(prefill_inputs(gshape, 0), gshape.dtype)
        gsteps = max(3, args.steps // 5)
        gplan, gms = run_prefill(gshape, hm, gt, gsteps, 2, two_streams=False)
        gms_attn = timed(lambda: hm.attn_with_kv(gt["q"], gplan.kv, gshape.Hkv, gshape.M,
                                                 gshape.W, gshape.rope_base, out=gplan.ya),
                         gsteps, 2)
        gfl = attn_flops(gshape)
        result["global_prefill"] = {
            "workload": gshape.name, "tokens_per_s": gshape.B * gshape.T / (gms * 1e-3),
            "ms_per_layer": gms, "attention_tflops": gfl / (gms_attn * 1e-3) / 1e12,
            "attention_frac_mfma": gfl / (gms_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del gt, gplan
        torch.cuda.empty_cache()
        sms, nl = run_stack(STACK, hm, 3, 1)
        result["stack"] = {"workload": STACK.name, "layers": nl,
                           "tokens_per_s_per_layer": STACK.B * STACK.T * nl / (sms * 1e-3),
                           "ms_per_stack": sms,
                           "inputs": "torch Philox generator on the device (same distributions)"}
        torch.cuda.empty_cache()
        kms, kl, kfl_mm, kfl_at = run_blocks(BLOCK_STACK, hm, BLOCK_STACK.layers, 3, 1)
        # the block stack's dominant kernel: a producer block's in-projection on its own
        gx, gw, gsegs = block_in_proj_operands(BLOCK_STACK)
        gouts = [torch.empty((gx.shape[0], c), dtype=torch.bfloat16, device="cuda") for c in gsegs]
        gms = timed(lambda: hm.linear(gx, gw, seg_cols=gsegs, outs=gouts), 10, 2)
        gfl = 2.0 * gx.shape[0] * gw.shape[0] * gx.shape[1]
        del gx, gw, gouts
        result["block_stack"] = {
            "workload": BLOCK_STACK.name + " (32 whole blocks, width 1600, FFN 5504)",
            "layers": kl, "ms_per_stack": kms,
            "tokens_per_s_per_layer": BLOCK_STACK.B * BLOCK_STACK.T * kl / (kms * 1e-3),
            "tokens_per_s": BLOCK_STACK.B * BLOCK_STACK.T / (kms * 1e-3),
            "tflops": (kfl_mm + kfl_at) / (kms * 1e-3) / 1e12,
            "frac_mfma": (kfl_mm + kfl_at) / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "linear_bf16_w4",
                         "launch": "a producer block's in-projection, 33024 x 1600 -> 5440",
                         "achieved": gfl / (gms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": gfl / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "algorithmic_flop_per_launch": gfl, "ms_per_launch": gms,
                         "traffic": traffic_from_profile(
                             LINEAR_SOURCES, "linear_bf16_w4.block-stack32-in-proj.pmc.txt")},
            "inputs": "torch Philox generator on the device (same distributions)"}
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, inp)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
