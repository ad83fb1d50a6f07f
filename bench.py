#!/usr/bin/env python3
"""Benchmark of the Hymba hybrid-head mixer core on one MI355X.

A step is one prefill pass of the 32-layer mixer stack (stack32-b2-t16512):
batch 2, 128 meta + 16384 tokens, 25 query heads x 64, 5 KV heads, SSM width
1600 x 16 states, conv width 4; layers 0, 15 and 31 global, the others a
1024-row sliding window with adjacent window layers sharing the producer's
prepared K/V; each layer is RoPE, the meta + window GQA attention, the causal
conv + selective scan branch and the branch norm and average, as three
launches on one stream; bf16 inputs with float32 accumulation, synthetic
seeded inputs resident in HBM.  `value` = prefill tokens/s per layer
(B * (M + N) rows * 32 layers / pass time), timed with HIP events over K
passes during which the library also records its launch boundaries.

Also reported on the same JSON line:
  roofline       the step's dominant kernel, the middle launch of a window layer
                 (attention | final scan pass), from the library's events around
                 it in every timed pass: attention FLOPs / time against the bf16
                 MFMA peak; the same for the three global layers (`global`);
  stack_kernels_us  mean time of each of the three launches per layer role;
  swa_prefill    one window layer (batch 1, 128 + 2048 rows): layer time, its
                 launches, and the attention kernel alone;
  cached_meta    that layer with the meta rows' K/V and SSM states cached;
  projections    the in- and out-projections around that layer;
  ssm_branch     the conv + scan branch alone against HBM and against the
                 measured ALU ceiling of its instruction mix (alu_probe);
  global_prefill the global layer (batch 4, 128 + 8192 rows);
  decode         one token for 64 sequences through an adjacent pair of layers
                 sharing a 128 + 1024-row KV cache: steps/s and HBM fraction with
                 the Infinity Cache flushed before each step (and warm);
  ragged_decode  the decode pair with one n_prev per sequence (warm);
  block, block_stack  whole Hymba blocks (norm, projections, mixer, norm, FFN):
                 one over the swa-prefill rows, 32 chained at the stack's size;
  cpu_baseline   the float64 CPU oracle on a bounded sample of the stack
                 (layers 0, 1, 2, 15, 30, 31), extrapolated, in the step's unit;
  cpu_baseline_decode  the oracle's decode step through the pair; swa_prefill and
                 global_prefill carry their own cpu_baseline (the whole layer, median
                 of 3; a sampled global layer, extrapolated).
HBM traffic (`traffic`) comes from the committed rocprofv3 counter summaries in
profiles/ (null once the kernel sources differ from those the counters were
taken with); `--counters` is the run those summaries are taken over.

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
               "hybrid_head_lm_amd/csrc/fused.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
STEP_SOURCES = ("hybrid_head_lm_amd/csrc/step.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
FUSED_SOURCES = ("hybrid_head_lm_amd/csrc/fused.hip", "hybrid_head_lm_amd/csrc/attn_dev.h",
                 "hybrid_head_lm_amd/csrc/ssm_dev.h", "hybrid_head_lm_amd/csrc/hm_common.h")
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


def blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max((d.get("num_threads") or 1) for d in info) if info else 1
    except Exception:
        return None


def _host(t):
    """A device tensor as float64 NumPy (bf16 widened exactly)."""
    import numpy as np
    return t.detach().float().cpu().numpy().astype(np.float64)


# sampled layers of the stack: global first, producer, consumer, global
# middle, unpaired window layer, global last
CPU_STACK_LAYERS = (0, 1, 2, 15, 30, 31)
CPU_QUERY_BLOCK = 512      # the oracle attention's own query-block size
CPU_SCAN_ROWS = 1024       # rows of the sequential scan timed per layer


def _oracle_layer_estimate(shape, window, q, k, v, part, prm):
    """Seconds of the oracle's prefill layer, from one 512-row query block of
    its attention (plus the K rotation it does once per call) and conv + scan +
    norm over the first CPU_SCAN_ROWS rows, extrapolated to all rows (the
    oracle scores every key of a row and masks, so each query block costs the
    same; the scan is sequential, linear in the rows)."""
    import numpy as np
    import oracle
    T, B = shape.T, shape.B
    n_blocks = -(-T // CPU_QUERY_BLOCK)
    qrows = np.arange(T // 2, T // 2 + CPU_QUERY_BLOCK)
    S = min(CPU_SCAN_ROWS, T)
    t0 = time.perf_counter()
    oracle.rope(k, np.arange(T), shape.rope_base)
    t_rope = time.perf_counter() - t0
    t0 = time.perf_counter()
    ya = oracle.attention(q, k, v, shape.M, window, shape.rope_base, rows=qrows)
    t_blk = time.perf_counter() - t0 - t_rope
    t0 = time.perf_counter()
    xc, _ = oracle.causal_conv1d(part["x"], prm["conv_w"], prm["conv_b"], None, True)
    ys, _ = oracle.selective_scan(xc, part["delta"], prm["A"], part["Bm"], part["Cm"],
                                  prm["D"], part["z"])
    t_ssm = time.perf_counter() - t0
    nr = min(S, len(qrows))
    t0 = time.perf_counter()
    oracle.branch_norm_mean(ya.reshape(B, len(qrows), -1)[:, :nr], ys[:, :nr],
                            prm["beta_a"], prm["beta_s"], shape.eps)
    t_norm = time.perf_counter() - t0
    return t_rope + n_blocks * max(t_blk, 0.0) + (T / S) * t_ssm + (T / nr) * t_norm


def _baseline_record(value, unit, sample, **extra):
    rec = {"value": value, "unit": unit, "cores": blas_threads() or 1,
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
           "kind": "oracle", "sample": sample}
    rec.update(extra)
    return rec


def cpu_baseline_layer(shape, inp, runs: int = 3):
    """The oracle's whole prefill layer on the workload's own host inputs,
    median of `runs` (small workloads)."""
    import oracle
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.mixer_prefill(inp, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
        ts.append(time.perf_counter() - t0)
    med = sorted(ts)[len(ts) // 2]
    return _baseline_record(shape.B * shape.T / med, "tokens/s",
                            f"{shape.name}: the whole layer, median of {runs} runs",
                            seconds_per_layer=med)


def cpu_baseline_layer_sampled(shape, inp):
    """The oracle's prefill layer on a bounded sample of a large workload
    (one query block and the first CPU_SCAN_ROWS rows), extrapolated."""
    S = min(CPU_SCAN_ROWS, shape.T)
    part = {n: inp[n][:, :S] for n in ("x", "delta", "Bm", "Cm", "z")}
    t0 = time.perf_counter()
    est = _oracle_layer_estimate(shape, shape.W, inp["q"], inp["k"], inp["v"], part, inp)
    wall = time.perf_counter() - t0
    return _baseline_record(
        shape.B * shape.T / est, "tokens/s",
        f"{shape.name}: the oracle attention over one {CPU_QUERY_BLOCK}-row query block plus "
        f"its K rotation, and conv + scan + norm over the first {S} rows, extrapolated to "
        f"{shape.T} rows; {wall:.1f} s of CPU work", seconds_per_layer_estimated=est)


def cpu_baseline_stack(shape, layers, roles):
    """The oracle (float64 NumPy, as it stands) on a bounded sample of the
    32-layer stack, extrapolated to the whole stack.

    Per sampled layer: the oracle attention over one 512-row query block (its
    own block size: it scores every key of a row and masks, so each block
    costs the same) and, timed separately, the rotation of all K rows it does
    once per call; the conv + selective scan over the first 1024 rows (the
    scan is sequential, linear in the rows); the branch norm-and-average of
    those rows.  Layer estimate = K rotation + (T / 512) blocks + (T / 1024) x
    (conv + scan + norm).  Stack estimate = 3 x mean(global layers) + 29 x
    mean(window layers).  Inputs are the stack's own device tensors copied to
    the host (the same bytes the GPU read)."""
    T = shape.T
    n_blocks = -(-T // CPU_QUERY_BLOCK)
    per_role = {"global": [], "window": []}
    t_all0 = time.perf_counter()
    for layer in CPU_STACK_LAYERS:
        window, src = roles[layer]
        t = layers[layer]
        q = _host(t["q"])
        k, v = _host(layers[src]["k"]), _host(layers[src]["v"])
        part = {n: _host(t[n][:, :CPU_SCAN_ROWS]) for n in ("x", "delta", "Bm", "Cm", "z")}
        prm = {n: _host(t[n]) for n in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s")}
        est = _oracle_layer_estimate(shape, window, q, k, v, part, prm)
        per_role["global" if window <= 0 else "window"].append(est)
        del q, k, v, part
    wall = time.perf_counter() - t_all0
    n_g = sum(1 for w, _ in roles if w <= 0)
    n_w = len(roles) - n_g
    t_stack = (n_g * sum(per_role["global"]) / len(per_role["global"])
               + n_w * sum(per_role["window"]) / len(per_role["window"]))
    return _baseline_record(
        shape.B * shape.T * len(roles) / t_stack, "tokens/s",
        (f"stack32-b2-t16512 layers {list(CPU_STACK_LAYERS)}: per layer the "
         f"oracle attention over one {CPU_QUERY_BLOCK}-row query block plus its "
         f"K rotation, and conv + scan + norm over the first {CPU_SCAN_ROWS} "
         f"rows; extrapolated to {n_blocks} blocks and {T} rows per layer, then "
         f"to {n_g} global + {n_w} window layers; {wall:.1f} s of CPU work; "
         "tokens/s per layer as the GPU value"),
        seconds_per_stack_estimated=t_stack)


def cpu_baseline_decode(shape, runs: int = 3):
    """The oracle's decode step through the producer / consumer pair on the
    decode workload (host inputs from the same generator), median of `runs`."""
    import oracle
    from workloads import decode_inputs
    d = decode_inputs(shape, 0)
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        ra = oracle.mixer_step(d["a"], d["k_cache"], d["v_cache"], shape.n_prev, shape.M,
                               shape.W, True, rope_base=shape.rope_base, eps=shape.eps)
        oracle.mixer_step(d["b"], ra["k_cache"], ra["v_cache"], shape.n_prev, shape.M, shape.W,
                          False, rope_base=shape.rope_base, eps=shape.eps)
        ts.append(time.perf_counter() - t0)
    med = sorted(ts)[len(ts) // 2]
    return {"value": 1.0 / med, "unit": "steps/s", "cores": blas_threads() or 1,
            "kind": "oracle",
            "sample": f"{runs} whole decode steps (both layers of the pair, B={shape.B}) of "
                      f"{shape.name}, median"}


def alu_probe(hm_dir: str):
    """Measured instruction rates of the vector ALU (libhm_probe.so): the
    transcendental rate, the fused multiply-add rate and the selective scan's
    single-pass mix (20 transcendental + 77 other VALU per token-channel), over
    the whole chip (2048 workgroups of 256 lanes, 8 waves per SIMD) timed with
    HIP events; and per SIMD at 1, 2, 4 and 8 waves, in shader-clock cycles
    (s_memtime against the 100 MHz s_memrealtime), which gives the clock the
    waves ran at and the issue rate per SIMD per cycle."""
    import ctypes
    import torch
    path = os.path.join(hm_dir, "libhm_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.hm_probe_alu.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.hm_probe_alu_counts.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int)]
    res = {}
    modes = ((0, "exp", 4000), (1, "fma", 4000), (2, "scan_mix", 60))
    # whole chip, 8 waves per SIMD
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * blocks * 4, dtype=torch.int64, device="cuda")
    for mode, name, iters in modes:
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        call = lambda: lib.hm_probe_alu(mode, ctypes.c_void_p(out.data_ptr()), blocks, 256,
                                        iters, ctypes.c_void_p(clk.data_ptr()), st)
        assert call() == 0
        ms = timed(call, 5, 2)
        c = clk.view(-1, 2).double()
        ghz = float((c[:, 0] / (c[:, 1] / 100e6)).median()) / 1e9
        tr, va = ctypes.c_int(), ctypes.c_int()
        lib.hm_probe_alu_counts(mode, ctypes.byref(tr), ctypes.byref(va))
        lanes = blocks * 256 * iters
        res[name] = {"trans_lane_ops_per_s": lanes * tr.value / (ms * 1e-3),
                     "valu_lane_ops_per_s": lanes * va.value / (ms * 1e-3), "ms": ms,
                     "clock_ghz": ghz}
    # the scan mix: 8 token-channels per lane per iteration
    res["scan_mix"]["token_channels_per_s"] = blocks * 256 * 60 * 8 / (res["scan_mix"]["ms"] * 1e-3)
    # per SIMD: one workgroup of w waves per CU... w waves on each SIMD of every CU:
    # 256 x 4 x w waves in 256-lane workgroups
    per_simd = {}
    for mode, name, iters in modes[:2]:
        for w in (1, 2, 4, 8):
            nb = 256 * w
            o = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
            ck = torch.zeros(2 * nb * 4, dtype=torch.int64, device="cuda")
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            assert lib.hm_probe_alu(mode, ctypes.c_void_p(o.data_ptr()), nb, 256, iters,
                                    ctypes.c_void_p(ck.data_ptr()), st) == 0
            torch.cuda.synchronize()
            c = ck.view(-1, 2).double()
            cyc = float(c[:, 0].median())
            # instructions one wave issues / its cycles x waves sharing the SIMD
            per_simd[f"{name}_w{w}"] = {"instr_per_cycle_per_simd": 8 * iters * w / cyc,
                                        "clock_ghz": float((c[:, 0] / (c[:, 1] / 100e6)).median()) / 1e9}
    res["per_simd"] = per_simd
    res["note"] = ("chip rates in lane-ops/s; per_simd: wave64 instructions issued per shader "
                   "cycle per SIMD with w waves on every SIMD (median wave), from s_memtime")
    return res


def run_prefill(shape, hm, t, steps, warmup, two_streams):
    import torch
    s2 = torch.cuda.Stream() if two_streams else None
    plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps,
                          want_states=False, stream2=s2)
    ms = timed(plan.run, steps, warmup)
    return plan, ms


def make_events(n: int):
    """n timing events, each created by one record() (the library records them
    again on its own stream)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs


def stack_layers(shape, hm):
    """Device inputs of the 32 layers (consumers without k, v) and the plan."""
    import torch
    from workloads import prefill_inputs_torch, stack_layer_roles
    roles = stack_layer_roles(shape)
    layers = []
    for layer, (_, src) in enumerate(roles):
        t = prefill_inputs_torch(shape, 0, layer, torch.device("cuda"))
        if src != layer:
            del t["k"], t["v"]
        layers.append(t)
    # one stream: every layer takes the fused three-launch sequence
    stack = hm.StackPlan(layers, roles, shape.M, shape.rope_base, shape.eps)
    return layers, roles, stack


def time_stack(stack, roles, steps, warmup, launches=("attn_final",)):
    """K passes of the stack with the library recording events around the
    given launches of every layer (distinct events per pass, read after the
    timed region).  Returns ms per pass (events around all passes), the mean
    microseconds of each of those launches per layer role (global / window)
    and the number of layers of each role."""
    import torch
    for _ in range(warmup):
        stack.run()
    n_l = len(roles)
    names = ("prep_agg", "attn_final", "norm_mean")
    want = [i for i in range(4) if any(names[j] in launches for j in (i - 1, i) if 0 <= j < 3)]
    evs = make_events(steps * n_l * len(want))
    per = []
    it = iter(evs)
    for k in range(steps):
        row = []
        for l in range(n_l):
            row.append([next(it) if i in want else None for i in range(4)])
        per.append(row)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for k in range(steps):
        stack.run(events=per[k])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kinds = {}
    for k in range(steps):
        for l, (w, src) in enumerate(roles):
            key = "global" if w <= 0 else "window"
            ev = per[k][l]
            d = kinds.setdefault(key, {n: [] for n in launches})
            for j, n in enumerate(names):
                if n in launches:
                    d[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    us = {key: {n: sum(v) / len(v) for n, v in d.items()} for key, d in kinds.items()}
    counts = {"global": sum(1 for w, _ in roles if w <= 0),
              "window": sum(1 for w, _ in roles if w > 0)}
    return ms, us, counts


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


def mfma_roofline(flop, us, kernel, launches, traffic=None, **extra):
    achieved = flop / (us * 1e-6) / 1e12
    d = {"bound": "mfma", "kernel": kernel, "launches": launches, "achieved": achieved,
         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
         "traffic": traffic, "algorithmic_flop_per_launch": flop, "us_per_launch": us}
    d.update(extra)
    return d


def layer_events(plan, steps, warmup):
    """Mean microseconds of the three launches of one layer, from the events
    the library records on its stream (distinct events per call)."""
    import torch
    for _ in range(warmup):
        plan.run()
    evs = make_events(4 * steps)
    torch.cuda.synchronize()
    for k in range(steps):
        plan.run(events=evs[4 * k:4 * k + 4])
    torch.cuda.synchronize()
    out = {"prep_agg": 0.0, "attn_final": 0.0, "norm_mean": 0.0}
    for k in range(steps):
        e = evs[4 * k:4 * k + 4]
        out["prep_agg"] += e[0].elapsed_time(e[1]) * 1e3 / steps
        out["attn_final"] += e[1].elapsed_time(e[2]) * 1e3 / steps
        out["norm_mean"] += e[2].elapsed_time(e[3]) * 1e3 / steps
    return out


def counters_run(hm, torch):
    """Calibration copies, then 3 launches each of the kernels whose counters
    profiles/ holds (for rocprofv3 --pmc runs; prints no JSON)."""
    from workloads import (BLOCK_STACK, DECODE_PAIR, GLOBAL_PREFILL, STACK, SWA_PREFILL,
                           decode_inputs, prefill_inputs, prefill_inputs_torch, to_device, with_)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    del src, dst
    # swa-prefill layer, its attention alone and its SSM branch alone
    shape = SWA_PREFILL
    t = to_device(prefill_inputs(shape, 0), shape.dtype)
    plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
    for _ in range(3):
        plan.run()
    for _ in range(3):
        hm.attn_with_kv(t["q"], plan.kv, shape.Hkv, shape.M, shape.W, shape.rope_base,
                        out=plan.ya)
    for _ in range(3):
        hm.conv_selective_scan(t["x"], t["conv_w"], t["conv_b"], t["delta"], t["A"], t["Bm"],
                               t["Cm"], t["D"], t["z"], out=plan.ys)
    del plan, t
    # global-prefill layer and its attention alone
    shape = GLOBAL_PREFILL
    t = to_device(prefill_inputs(shape, 0), shape.dtype)
    plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps)
    for _ in range(3):
        plan.run()
    for _ in range(3):
        hm.attn_with_kv(t["q"], plan.kv, shape.Hkv, shape.M, shape.W, shape.rope_base,
                        out=plan.ya)
    del plan, t
    # one window layer and one global layer at the stack's size
    for w in (STACK.W, 0):
        shape = with_(STACK, W=w)
        t = prefill_inputs_torch(shape, 0, 1 if w > 0 else 0, torch.device("cuda"))
        plan = hm.PrefillPlan(t, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps,
                              want_states=False)
        for _ in range(3):
            plan.run()
        del plan, t
    torch.cuda.empty_cache()
    # decode pair
    dshape = DECODE_PAIR
    d = to_device(decode_inputs(dshape, 0), dshape.dtype)
    pa = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W)
    pb = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W)
    for _ in range(3):
        pa.run()
        pb.run()
    del pa, pb, d
    # the block stack's in-projection
    x, w, segs = block_in_proj_operands(BLOCK_STACK)
    outs = [torch.empty((x.shape[0], c), dtype=torch.bfloat16, device="cuda") for c in segs]
    for _ in range(3):
        hm.linear(x, w, seg_cols=segs, outs=outs)
    torch.cuda.synchronize()
    print("counters run done: 3 copies of", COPY_BYTES, "bytes, then 3 each of: swa-prefill "
          "layer, its attention, its SSM branch; global-prefill layer, its attention; a window "
          "and a global layer of the stack; the decode pair; the block-stack in-projection")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true",
                    help="skip the block and block-stack lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="only a 256 MiB device copy (calibration) and the kernels whose "
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
                           SWA_PREFILL, decode_inputs, prefill_inputs, to_device, with_)

    torch.cuda.set_device(0)
    if args.counters:
        counters_run(hm, torch)
        return

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ the step:
    # one pass of the 32-layer stack, the library recording its launch
    # boundaries; a second, uninstrumented timing beside it
    shape = STACK
    layers, roles, stack = stack_layers(shape, hm)
    log("stack inputs ready")
    ms, us, counts = time_stack(stack, roles, args.steps, args.warmup)
    ms_plain = timed(stack.run, args.steps, 1)
    _, us_all, _ = time_stack(stack, roles, max(3, args.steps // 4), 1,
                              launches=("prep_agg", "attn_final", "norm_mean"))
    log(f"stack {ms:.3f} ms per pass (uninstrumented {ms_plain:.3f})")
    n_layers = len(roles)
    rows = shape.B * shape.T
    fl_w = attn_flops(with_(shape, W=shape.W))
    fl_g = attn_flops(with_(shape, W=0))
    fused_traffic = traffic_from_profile(FUSED_SOURCES, "prefill_attn_final.stack32-window.pmc.txt")
    fused_traffic_g = traffic_from_profile(FUSED_SOURCES,
                                           "prefill_attn_final.stack32-global.pmc.txt")
    kern_ms = {k: sum(counts[r] * us[r][k] for r in us) / 1e3 for k in ("attn_final",)}
    result = {
        "metric": "hybrid-mixer prefill tokens/s per layer + decode steps/s; % MFMA/HBM roofline",
        "value": rows * n_layers / (ms * 1e-3),
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
        "config": {"workload": shape.name, "layers": n_layers,
                   "global_layers": list(shape.global_layers), "batch": shape.B,
                   "meta_tokens": shape.M, "tokens": shape.N, "rows": shape.T,
                   "q_heads": shape.Hq, "kv_heads": shape.Hkv, "head_dim": shape.Dh,
                   "window": shape.W, "ssm_width": shape.Di, "ssm_states": shape.Ns,
                   "conv": shape.K,
                   "kv_sharing": "window layers paired (1,2)..(13,14), (16,17)..(28,29); "
                                 "layer 30 alone",
                   "step": "one pass of the 32 mixer layers, three launches per layer on one "
                           "stream; value = rows x layers / pass time (tokens/s per layer)"},
        "ms_per_step_uninstrumented": ms_plain,
        "timing": "HIP events around the K timed passes; inside them the library records "
                  "two more events per layer around its middle launch (the roofline); "
                  "ms_per_step_uninstrumented is the same stack timed without them",
        "roofline": mfma_roofline(
            fl_w, us["window"]["attn_final"], "prefill_attn_final",
            f"the {counts['window']} window layers of each pass (attention | final scan "
            "pass of the SSM branch in one launch; FLOPs count the attention only)",
            traffic=fused_traffic,
            final_scan_bytes_per_launch=scan_bytes(shape),
            share_of_step_all_layers=kern_ms["attn_final"] / ms,
            timing="HIP events the library records on its stream around this launch in every "
                   "layer of every timed pass",
            **{"global": mfma_roofline(fl_g, us["global"]["attn_final"], "prefill_attn_final",
                                       f"the {counts['global']} global layers of each pass",
                                       traffic=fused_traffic_g)}),
        "stack_kernels_us": us_all,
        "stack_kernels_ms_per_pass": {
            f"{k}_{r}": counts[r] * us_all[r][k] / 1e3 for r in us_all for k in us_all[r]},
        "stack_kernels_note": "from separate passes with events around all three launches "
                              "of every layer, after the timed region",
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (stack sample)")
        result["cpu_baseline"] = cpu_baseline_stack(shape, layers, roles)
    del stack, layers
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ swa-prefill layer
    log("swa-prefill layer")
    sshape = SWA_PREFILL
    inp = prefill_inputs(sshape, 0)
    t = to_device(inp, sshape.dtype)
    lsteps = max(50, args.steps)
    plan, ms_l = run_prefill(sshape, hm, t, lsteps, 10, two_streams=False)
    sclk = []
    layer_dist = step_percentiles(plan.run, 200, while_busy=lambda: sample_sclk(sclk))
    cur = [c for c, _ in sclk if c is not None]
    _, ms_two = run_prefill(sshape, hm, t, lsteps, 10, two_streams=True)
    lev = layer_events(plan, lsteps, 5)
    fl = attn_flops(sshape)
    ms_attn = timed(lambda: hm.attn_with_kv(t["q"], plan.kv, sshape.Hkv, sshape.M, sshape.W,
                                            sshape.rope_base, out=plan.ya), lsteps, 10)
    ms_ssm = timed(lambda: hm.conv_selective_scan(t["x"], t["conv_w"], t["conv_b"], t["delta"],
                                                  t["A"], t["Bm"], t["Cm"], t["D"], t["z"],
                                                  out=plan.ys), lsteps, 10)
    ms_norm = timed(lambda: hm.branch_norm_mean(plan.ya, plan.ys, t["beta_a"], t["beta_s"],
                                                sshape.eps, out=plan.out), lsteps, 10)
    result["swa_prefill"] = {
        "workload": sshape.name, "tokens_per_s": sshape.B * sshape.T / (ms_l * 1e-3),
        "ms_per_layer": ms_l, "layer_step_us": layer_dist,
        "kernels_us": lev,
        "roofline": mfma_roofline(fl, lev["attn_final"], "prefill_attn_final",
                                  "the layer's middle launch (attention | final scan)"),
        "attention_alone": mfma_roofline(
            fl, ms_attn * 1e3, "attn_fwd_bf16", "attention alone over the prepared K/V",
            traffic=traffic_from_profile(ATTN_SOURCES,
                                         "attn_fwd_bf16.swa-prefill-b1-t2176.pmc.txt")),
        "breakdown_ms": {"layer_one_stream": ms_l, "layer_two_streams": ms_two,
                         "attention_kernel": ms_attn, "ssm_branch": ms_ssm, "norm_mean": ms_norm},
        "sclk_mhz": {"max_sampled": max(cur) if cur else None,
                     "highest_level": sclk[0][1] if sclk else None,
                     "note": "the driver's current-clock line, read 12 times 1 ms apart while "
                             "layer calls run: an average including idle time"}}
    if not args.no_cpu_baseline:
        log("cpu baseline (swa-prefill layer)")
        result["swa_prefill"]["cpu_baseline"] = cpu_baseline_layer(sshape, inp)

    # the same layer with the meta tokens cached (real-token rows only)
    from workloads import cached_meta_inputs
    _, ctok, cmeta = cached_meta_inputs(sshape, 0)
    ct = to_device(ctok, sshape.dtype)
    cmk = to_device({"k": cmeta["k"], "v": cmeta["v"]}, sshape.dtype)
    cst = torch.zeros((sshape.B, sshape.Di, sshape.K - 1), dtype=torch.float32, device="cuda")
    ch0 = torch.zeros((sshape.B, sshape.Di, sshape.Ns), dtype=torch.float32, device="cuda")
    cplan = hm.PrefillPlan(ct, sshape.M, sshape.W, rope_base=sshape.rope_base, eps=sshape.eps,
                           want_states=False, meta={"k": cmk["k"], "v": cmk["v"]},
                           conv_state_in=cst, h0=ch0)
    ms_cached = timed(cplan.run, lsteps, 10)
    result["cached_meta"] = {"workload": sshape.name + " with the 128 meta rows cached",
                             "real_tokens_per_s": sshape.B * sshape.N / (ms_cached * 1e-3),
                             "ms_per_layer": ms_cached,
                             "full_layer_real_tokens_per_s": sshape.B * sshape.N / (ms_l * 1e-3)}
    del cplan, ct, cmk

    # the projections around the layer
    gen = torch.Generator(device="cuda").manual_seed(3)
    d_model = sshape.Hq * sshape.Dh
    segs = [sshape.Hq * sshape.Dh, sshape.Hkv * sshape.Dh, sshape.Hkv * sshape.Dh, sshape.Di,
            sshape.Di]
    px = torch.randn(sshape.B * sshape.T, d_model, device="cuda", generator=gen).bfloat16()
    pw_in = (torch.randn(sum(segs), d_model, device="cuda", generator=gen)
             / d_model ** 0.5).bfloat16()
    pw_out = (torch.randn(d_model, sshape.Di, device="cuda", generator=gen)
              / sshape.Di ** 0.5).bfloat16()
    pouts = [torch.empty(sshape.B * sshape.T, c, dtype=torch.bfloat16, device="cuda")
             for c in segs]
    py = torch.empty(sshape.B * sshape.T, d_model, dtype=torch.bfloat16, device="cuda")
    ms_in = timed(lambda: hm.linear(px, pw_in, seg_cols=segs, outs=pouts), lsteps, 10)
    ms_out = timed(lambda: hm.linear(pouts[3], pw_out, outs=[py]), lsteps, 10)
    fl_in = 2.0 * sshape.B * sshape.T * sum(segs) * d_model
    fl_out = 2.0 * sshape.B * sshape.T * d_model * sshape.Di
    result["projections"] = {
        "workload": sshape.name + " in-projection 1600 -> Q, K, V, x, z (5440) and "
                                  "out-projection 1600 -> 1600, bf16",
        "in_proj": mfma_roofline(fl_in, ms_in * 1e3, "linear_bf16_w4", "one call"),
        "out_proj": mfma_roofline(fl_out, ms_out * 1e3, "linear_bf16", "one call")}
    del px, pw_in, pw_out, pouts, py

    # ------------------------------------------------------------ SSM branch and ALU ceiling
    log("ssm branch and ALU probe")
    probe = alu_probe(os.path.dirname(hm.LIB_PATH))
    tc_ssm = sshape.B * sshape.T * sshape.Di
    bound_tc = probe["scan_mix"]["token_channels_per_s"] if probe else None
    result["ssm_branch"] = {
        "workload": sshape.name + ": conv + selective scan alone (hm_conv_selective_scan)",
        "bound": "hbm", "achieved": scan_bytes(sshape) / (ms_ssm * 1e-3) / 1e9,
        "peak": PEAK_HBM_GBPS, "unit": "GB/s",
        "frac": scan_bytes(sshape) / (ms_ssm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "ms": ms_ssm,
        "traffic": traffic_from_profile(SSM_SOURCES, "ssm-branch.swa-prefill-b1-t2176.pmc.txt",
                                        "hbm_bytes_per_call"),
        "alu": {"bound": "alu", "unit": "token-channels/s",
                "achieved": tc_ssm / (ms_ssm * 1e-3), "peak": bound_tc,
                "frac": (tc_ssm / (ms_ssm * 1e-3) / bound_tc) if bound_tc else None,
                "peak_source": "measured: the scan's single-pass instruction mix per "
                               "token-channel (20 transcendental + 77 other VALU) run on every "
                               "SIMD (alu_probe.scan_mix)",
                "valu_per_token_channel": SCAN_VALU_PER_TC,
                "transcendental_per_token_channel": SCAN_TRANS_PER_TC}}
    result["alu_probe"] = probe
    del plan, t
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ global-prefill layer
    log("global-prefill layer")
    gshape = GLOBAL_PREFILL
    ginp = prefill_inputs(gshape, 0)
    gt = to_device(ginp, gshape.dtype)
    gsteps = max(5, args.steps // 2)
    gplan, gms = run_prefill(gshape, hm, gt, gsteps, 2, two_streams=False)
    gev = layer_events(gplan, gsteps, 1)
    gms_attn = timed(lambda: hm.attn_with_kv(gt["q"], gplan.kv, gshape.Hkv, gshape.M, gshape.W,
                                             gshape.rope_base, out=gplan.ya), gsteps, 2)
    gfl = attn_flops(gshape)
    result["global_prefill"] = {
        "workload": gshape.name, "tokens_per_s": gshape.B * gshape.T / (gms * 1e-3),
        "ms_per_layer": gms, "kernels_us": gev,
        "roofline": mfma_roofline(gfl, gev["attn_final"], "prefill_attn_final",
                                  "the layer's middle launch (attention | final scan)"),
        "attention_alone": mfma_roofline(gfl, gms_attn * 1e3, "attn_fwd_bf16",
                                         "attention alone over the prepared K/V")}
    if not args.no_cpu_baseline:
        log("cpu baseline (global-prefill sample)")
        result["global_prefill"]["cpu_baseline"] = cpu_baseline_layer_sampled(gshape, ginp)
    del gt, gplan, ginp
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode
    log("decode")
    dshape = DECODE_PAIR
    d = to_device(decode_inputs(dshape, 0), dshape.dtype)
    pa = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W,
                     rope_base=dshape.rope_base, eps=dshape.eps)
    pb = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], dshape.n_prev, dshape.M, dshape.W,
                     rope_base=dshape.rope_base, eps=dshape.eps)

    def decode_step():
        pa.run()
        pb.run()
    dsteps = max(50, args.steps)
    ms_dec = timed(decode_step, dsteps, 10)
    dbytes = decode_bytes(dshape)
    # cold: before every step a 512 MB write evicts the pair's cache and states
    # from the 256 MB Infinity Cache, as the other layers of a model would, and a
    # 1 GB read then leaves the cache holding clean lines
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush_rd = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cold = []
    for i in range(10 + dsteps):
        flush.fill_(i & 0xFF)
        flush_rd.max()
        e0.record()
        decode_step()
        e1.record()
        torch.cuda.synchronize()
        if i >= 10:
            cold.append(e0.elapsed_time(e1))
    ms_dec_cold = sum(cold) / len(cold)
    del flush, flush_rd
    result["decode"] = {
        "workload": dshape.name, "steps_per_s": 1e3 / ms_dec_cold,
        "tokens_per_s": dshape.B * 1e3 / ms_dec_cold, "ms_per_step": ms_dec_cold,
        "cache": "cold (Infinity Cache flushed before every step: 512 MB written, then 1 GB "
                 "read)",
        "roofline": {"bound": "hbm", "achieved": dbytes / (ms_dec_cold * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": dbytes / (ms_dec_cold * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                     "algorithmic_bytes_per_step": dbytes,
                     "traffic": traffic_from_profile(
                         STEP_SOURCES, "step-pair.decode-pair-b64-cache1152.pmc.txt",
                         "hbm_bytes_per_step")},
        "warm": {"steps_per_s": 1e3 / ms_dec, "ms_per_step": ms_dec,
                 "hbm_frac": dbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                 "note": "back-to-back steps; the 222 MB of the pair stay in the 256 MB "
                         "Infinity Cache"}}
    nps = np.random.default_rng(5).integers(0, 2048, size=dshape.B).astype(np.int32)
    npt = torch.from_numpy(nps).cuda()
    ra_plan = hm.StepPlan(d["a"], d["k_cache"], d["v_cache"], int(nps.max()), dshape.M, dshape.W,
                          rope_base=dshape.rope_base, eps=dshape.eps, n_prev_seq=npt)
    rb_plan = hm.StepPlan(d["b"], d["k_cache"], d["v_cache"], int(nps.max()), dshape.M, dshape.W,
                          rope_base=dshape.rope_base, eps=dshape.eps, n_prev_seq=npt)

    def ragged_step():
        ra_plan.run()
        rb_plan.run()
    ms_rag = timed(ragged_step, dsteps, 10)
    rag_bytes = decode_bytes(dshape, nps)
    result["ragged_decode"] = {
        "workload": dshape.name + " with n_prev per sequence uniform over 0..2047 (seeded)",
        "steps_per_s": 1e3 / ms_rag, "ms_per_step": ms_rag,
        "hbm_frac": rag_bytes / (ms_rag * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": rag_bytes, "cache": "warm (back-to-back steps)"}
    del ra_plan, rb_plan, pa, pb, d
    if not args.no_cpu_baseline:
        log("cpu baseline (decode)")
        result["cpu_baseline_decode"] = cpu_baseline_decode(dshape)
    torch.cuda.empty_cache()

    if not args.quick:
        log("blocks")
        bshape = BLOCK_SWA
        bms, _, bfl_mm, bfl_at = run_blocks(bshape, hm, 1, lsteps, 10)
        result["block"] = {
            "workload": bshape.name + " (width 1600, FFN 5504; norm, projections, mixer, "
                                      "norm, FFN)",
            "tokens_per_s": bshape.B * bshape.T / (bms * 1e-3), "ms_per_block": bms,
            "mixer_ms": ms_l, "matmul_tflop": bfl_mm / 1e12,
            "tflops": (bfl_mm + bfl_at) / (bms * 1e-3) / 1e12,
            "frac_mfma": (bfl_mm + bfl_at) / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        torch.cuda.empty_cache()
        kms, kl, kfl_mm, kfl_at = run_blocks(BLOCK_STACK, hm, BLOCK_STACK.layers, 5, 1)
        gx, gw, gsegs = block_in_proj_operands(BLOCK_STACK)
        gouts = [torch.empty((gx.shape[0], c), dtype=torch.bfloat16, device="cuda")
                 for c in gsegs]
        kgms = timed(lambda: hm.linear(gx, gw, seg_cols=gsegs, outs=gouts), 10, 2)
        kgfl = 2.0 * gx.shape[0] * gw.shape[0] * gx.shape[1]
        del gx, gw, gouts
        result["block_stack"] = {
            "workload": BLOCK_STACK.name + " (32 whole blocks, width 1600, FFN 5504)",
            "layers": kl, "ms_per_stack": kms,
            "tokens_per_s_per_layer": BLOCK_STACK.B * BLOCK_STACK.T * kl / (kms * 1e-3),
            "tokens_per_s": BLOCK_STACK.B * BLOCK_STACK.T / (kms * 1e-3),
            "tflops": (kfl_mm + kfl_at) / (kms * 1e-3) / 1e12,
            "frac_mfma": (kfl_mm + kfl_at) / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "roofline": mfma_roofline(
                kgfl, kgms * 1e3, "linear_bf16_w4",
                "a producer block's in-projection, 33024 x 1600 -> 5440",
                traffic=traffic_from_profile(LINEAR_SOURCES,
                                             "linear_bf16_w4.block-stack32-in-proj.pmc.txt")),
            "inputs": "torch Philox generator on the device (same distributions)"}
        torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
