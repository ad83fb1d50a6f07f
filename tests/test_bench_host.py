"""Host-side checks of bench.py (no GPU): the work counts its roofline
fractions divide by, the refusal of more than one GPU, the counter-summary
reader and the oracle CPU baselines on small shapes.

The FLOP and byte counts are pinned to sums taken over the oracle's own mask
and to the figures the attention and decode definitions give by hand, not to
bench.py's formulas.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from workloads import DECODE_PAIR, GLOBAL_PREFILL, STACK, SWA_PREFILL, with_, prefill_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("T,M,W", [(64, 4, 16), (300, 16, 100), (257, 3, 0), (130, 128, 1)])
def test_attn_flops_counts_visible_pairs(T, M, W):
    # 4 Dh FLOP (QK^T and PV) per visible (query, key) pair, per query head and sequence
    shape = with_(SWA_PREFILL, B=3, M=M, N=T - M, W=W, Hq=5, Dh=16, Di=80)
    pairs = int(oracle.mask(T, M, W).sum())
    assert bench.attn_flops(shape) == 4 * 16 * 5 * 3 * pairs


def test_attn_flops_of_the_measured_workloads():
    # swa-prefill: sum_i min(i+1, 1152) over 2176 rows = 1 843 776 pairs per head
    assert bench.attn_flops(SWA_PREFILL) == 4 * 64 * 25 * 1 * 1_843_776
    # a global layer of the stack: 16512 * 16513 / 2 pairs per head and sequence
    g = with_(STACK, W=0)
    assert bench.attn_flops(g) == 4 * 64 * 25 * 2 * (16512 * 16513 // 2)
    assert bench.attn_flops(GLOBAL_PREFILL) == 4 * 64 * 25 * 4 * (8320 * 8321 // 2)


def test_decode_bytes_of_the_pair():
    # per layer: 64 sequences x 1152 visible rows x 5 KV heads x 64 dims x (K, V) x 2 B,
    # SSM state [64, 1600, 16] f32 and conv state [64, 1600, 3] f32 read and written,
    # q [64, 25, 64], x / delta / z / out [64, 1600] bf16, B / C [64, 16] bf16; the
    # producer also reads k_new, v_new [64, 5, 64] bf16 and writes them to the cache
    B, Di = 64, 1600
    layer = (B * 1152 * 5 * 64 * 2 * 2 + B * Di * 16 * 4 * 2 + B * Di * 3 * 4 * 2
             + B * 25 * 64 * 2 + B * Di * 2 * 4 + B * 16 * 2 * 2)
    assert bench.decode_bytes(DECODE_PAIR) == 2 * layer + B * 5 * 64 * 2 * 2 * 2
    assert abs(bench.decode_bytes(DECODE_PAIR) - 222.09e6) < 0.01e6


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_summaries_parse():
    # every committed summary either matches the current kernel sources (a
    # positive byte count) or is reported stale (None); none breaks the reader
    names = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith(".pmc.txt"))
    assert names
    for name in names:
        v = bench.traffic_from_profile(("bench.py",), name)
        assert v is None or v > 0
    assert bench.traffic_from_profile(("bench.py",), "no-such-summary.txt") is None


def test_cpu_baselines_on_small_shapes():
    small = with_(SWA_PREFILL, N=200, M=8, W=64, Hq=2, Hkv=1, Di=128)
    rec = bench.cpu_baseline_layer(small, prefill_inputs(small, 0), runs=1)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and "sample" in rec
    big = with_(GLOBAL_PREFILL, B=1, N=1400, M=8, Hq=2, Hkv=1, Di=128)
    rec = bench.cpu_baseline_layer_sampled(big, prefill_inputs(big, 0))
    assert rec["value"] > 0 and rec["seconds_per_layer_estimated"] > 0
    assert str(big.T) in rec["sample"]
