"""Write the profiles/*.txt summaries from rocprofv3's CSV output.

Usage (R = repository root, OUT = any scratch directory; the GPU steps run on
the MI355X machine from /tmp with TMPDIR=/tmp, the last one anywhere):

    rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o bench \\
        -- python3 $R/bench.py > $OUT/bench_kt.json
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o run \\
        -- python3 $R/bench.py --counters
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o run \\
        -- python3 $R/bench.py --counters
    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU \\
        SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_INSTS_LDS GRBM_GUI_ACTIVE \\
        --output-format csv -d $OUT/pmc_sq -o run -- python3 $R/bench.py --counters
    python3 $R/bench_profiles.py $OUT

(each counter pass under `timeout -s KILL 200`: a pass asking for more
counters than the hardware collects at once hangs instead of failing).

What it writes:
  * one counter summary per kernel and workload: HBM bytes per launch from
    FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for
    the 256 MiB device copies `bench.py --counters` runs first (their bytes are
    known), the algorithmic bytes beside them, and the MFMA-busy / VALU-issue
    fractions from the SQ pass; the last lines are read back by bench.py,
    which takes the byte figure only while the sha256 of the kernel sources it
    lists still matches;
  * the kernel-trace summary of the default bench run (mean duration per
    kernel and launch grid), with bench.py's own event timings of that run.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 268435456          # one calibration copy: 256 MiB read and 256 MiB written
COPY_GRID = 131072

CMD = {
    "fetch": "timeout -s KILL 200 rocprofv3 --pmc FETCH_SIZE --output-format csv "
             "-d $OUT/pmc_fetch -o run -- python3 $R/bench.py --counters",
    "write": "timeout -s KILL 200 rocprofv3 --pmc WRITE_SIZE --output-format csv "
             "-d $OUT/pmc_write -o run -- python3 $R/bench.py --counters",
    "sq": "timeout -s KILL 200 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
          "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_INSTS_LDS "
          "GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_sq -o run -- python3 $R/bench.py "
          "--counters",
    "kt": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o bench -- "
          "python3 $R/bench.py > $OUT/bench_kt.json",
    "sum": "python3 $R/bench_profiles.py $OUT",
}
HEAD = """# Commands (on the MI355X machine, from /tmp with TMPDIR=/tmp; R = repository root,
# OUT = a scratch directory):
#   {fetch}
#   {write}
#   {sq}
#   {sum}
# `bench.py --counters` runs 3 device copies of 256 MiB (__amd_rocclr_copyBuffer, the
# calibration: 268435456 bytes read and written each), then 3 launches each of: the
# swa-prefill layer, its attention alone, its SSM branch alone; the global-prefill layer,
# its attention alone; one window and one global layer at the stack's size; the decode
# pair; the block stack's in-projection.""".format(**CMD)

FUSED = ("hybrid_head_lm_amd/csrc/fused.hip", "hybrid_head_lm_amd/csrc/attn_dev.h",
         "hybrid_head_lm_amd/csrc/ssm_dev.h", "hybrid_head_lm_amd/csrc/hm_common.h")
ATTN = ("hybrid_head_lm_amd/csrc/attn_dev.h", "hybrid_head_lm_amd/csrc/attn.hip",
        "hybrid_head_lm_amd/csrc/hm_common.h")
SSM = ("hybrid_head_lm_amd/csrc/ssm_dev.h", "hybrid_head_lm_amd/csrc/ssm.hip",
       "hybrid_head_lm_amd/csrc/fused.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
STEP = ("hybrid_head_lm_amd/csrc/step.hip", "hybrid_head_lm_amd/csrc/hm_common.h")
LIN = ("hybrid_head_lm_amd/csrc/linear_w4.hip", "hybrid_head_lm_amd/csrc/linear_dev.h",
       "hybrid_head_lm_amd/csrc/linear.hip", "hybrid_head_lm_amd/csrc/hm_common.h")


def sha(paths) -> str:
    """The source fingerprint bench.py compares (same function as its own)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kname(n: str) -> str:
    n = n.replace("(anonymous namespace)::", "")
    n = re.sub(r"^void ", "", n)
    m = re.match(r"([A-Za-z_0-9:]+(<[^()]*>)?)", n)
    return m.group(1) if m else n[:50]


def load_pmc(path):
    """Counter values per dispatch and (kernel, grid threads, workgroup, us) per dispatch."""
    rows = collections.defaultdict(dict)
    meta = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            rows[did][r["Counter_Name"]] = float(r["Counter_Value"])
            meta[did] = (kname(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Workgroup_Size"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return rows, meta


def ordered(meta, kern, grid):
    return [d for d in sorted(meta) if meta[d][0] == kern and meta[d][1] == grid]


class Counters:
    """The three counter passes of `bench.py --counters` under one directory."""

    def __init__(self, out_dir: str):
        self.fetch, self.fmeta = load_pmc(os.path.join(out_dir, "pmc_fetch", "run_counter_collection.csv"))
        self.write, self.wmeta = load_pmc(os.path.join(out_dir, "pmc_write", "run_counter_collection.csv"))
        self.sq, self.smeta = load_pmc(os.path.join(out_dir, "pmc_sq", "run_counter_collection.csv"))
        cf = [self.fetch[d]["FETCH_SIZE"] for d in ordered(self.fmeta, "__amd_rocclr_copyBuffer", COPY_GRID)]
        cw = [self.write[d]["WRITE_SIZE"] for d in ordered(self.wmeta, "__amd_rocclr_copyBuffer", COPY_GRID)]
        if not cf or not cw:
            raise SystemExit("no calibration copies in the counter passes")
        self.sf = COPY_BYTES / (sum(cf) / len(cf) * 1024)
        self.sw = COPY_BYTES / (sum(cw) / len(cw) * 1024)
        self.cal = (f"# counter        copy (KiB/dispatch)   scale = known/counted\n"
                    f"# FETCH_SIZE      {sum(cf)/len(cf):12.1f}          {self.sf:.4f}\n"
                    f"# WRITE_SIZE      {sum(cw)/len(cw):12.1f}          {self.sw:.4f}")

    def traffic(self, kern, grid, pick=None):
        """Counted KiB per dispatch (fetch, write) and the scaled bytes per dispatch."""
        fd, wd = ordered(self.fmeta, kern, grid), ordered(self.wmeta, kern, grid)
        if pick is not None:
            fd, wd = [fd[i] for i in pick], [wd[i] for i in pick]
        if not fd or not wd:
            raise SystemExit(f"no dispatches of {kern} with grid {grid} in the counter passes")
        f = [self.fetch[d]["FETCH_SIZE"] for d in fd]
        w = [self.write[d]["WRITE_SIZE"] for d in wd]
        return f, w, sum(f) / len(f) * 1024 * self.sf, sum(w) / len(w) * 1024 * self.sw

    def sq_block(self, dids, label):
        """MFMA-busy and VALU-issue fractions of the given dispatches (mean).  The
        busy fractions need GRBM_GUI_ACTIVE to span the kernel alone, which it
        does not for launches of a few tens of microseconds (the clock it implies
        then exceeds the chip's maximum): none are given for those."""
        vals = collections.defaultdict(list)
        for d in dids:
            v = self.sq[d]
            cyc = v["GRBM_GUI_ACTIVE"] / 8.0          # summed over the 8 XCDs
            vals["clock_ghz"].append(cyc / (self.smeta[d][3] * 1e3))
            vals["mfma_busy"].append(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024))
            vals["valu_active"].append(v["SQ_ACTIVE_INST_VALU"] * 4 / (cyc * 1024))
            vals["valu_insts"].append(v["SQ_INSTS_VALU"])
            vals["trans_insts"].append(v["SQ_INSTS_VALU_TRANS_F32"])
            vals["mfma_insts"].append(v["SQ_INSTS_MFMA"])
            vals["lds_insts"].append(v["SQ_INSTS_LDS"])
            vals["us"].append(self.smeta[d][3])
        m = {k: sum(x) / len(x) for k, x in vals.items()}
        out = [f"# {label}: {len(dids)} dispatches under the counter pass, mean {m['us']:.1f} us each"]
        if m["clock_ghz"] > 2.45:
            out.append(f"#   cycles = GRBM_GUI_ACTIVE / 8 gives {m['clock_ghz']:.2f} GHz, above the 2.4 GHz "
                       "maximum: for a kernel this short the counter does not cover the kernel alone, "
                       "so no busy fractions are derived")
        else:
            out.append(f"#   cycles = GRBM_GUI_ACTIVE / 8 (summed over the 8 XCDs) -> clock "
                       f"{m['clock_ghz']:.2f} GHz during the kernel")
            out.append(f"#   MFMA busy   = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)       = {m['mfma_busy']:.3f}")
            out.append(f"#   VALU issue  = SQ_ACTIVE_INST_VALU x 4 / (cycles x 1024 SIMDs)         = {m['valu_active']:.3f}")
        out.append(f"#   instructions per dispatch: VALU {m['valu_insts']:.4g} (of which transcendental "
                   f"{m['trans_insts']:.4g}), MFMA {m['mfma_insts']:.4g}, LDS {m['lds_insts']:.4g}")
        return out, m


def write_single(c: Counters, fname, title, kern, grid, pick, srcs, alg_desc, alg_bytes,
                 extra=None):
    """Summary of one kernel's launches (`pick`: which of the matching dispatches)."""
    f, w, fb, wb = c.traffic(kern, grid, pick)
    sd = ordered(c.smeta, kern, grid)
    if pick is not None:
        sd = [sd[i] for i in pick]
    sqo, m = c.sq_block(sd, kern)
    lines = [f"# {title}", "#", HEAD, "#", c.cal, "#",
             f"# {kern} (KiB/dispatch): FETCH_SIZE " + ", ".join(f"{x:.1f}" for x in f) +
             "; WRITE_SIZE " + ", ".join(f"{x:.1f}" for x in w),
             f"# scaled HBM bytes per launch: read {fb/1e6:.2f} MB + written {wb/1e6:.2f} MB = {(fb+wb)/1e6:.2f} MB",
             f"# algorithmic bytes per launch: {alg_desc} = {alg_bytes/1e6:.2f} MB "
             f"(counted / algorithmic = {(fb+wb)/alg_bytes:.2f})", "#"] + sqo
    if extra:
        lines += ["#"] + [f"# {e}" for e in extra]
    busy = m["clock_ghz"] <= 2.45
    lines += ["# The figures below are read by bench.py; source_sha256_16 is the first 16 hex digits of",
              "# the sha256 over " + ", ".join(srcs) + " (in that order) the counters were taken with.",
              f"kernel = {kern}", f"grid_threads = {grid}", f"source_sha256_16 = {sha(srcs)}",
              f"fetch_bytes_per_launch = {fb:.0f}", f"write_bytes_per_launch = {wb:.0f}",
              f"hbm_bytes_per_launch = {fb + wb:.0f}",
              f"mfma_busy = {m['mfma_busy']:.4f}" if busy else "mfma_busy = n/a",
              f"valu_issue = {m['valu_active']:.4f}" if busy else "valu_issue = n/a",
              f"clock_ghz = {m['clock_ghz']:.3f}" if busy else "clock_ghz = n/a"]
    with open(os.path.join(PROFILES, fname), "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("wrote", fname, f"{(fb + wb)/1e6:.1f} MB")


def write_multi(c: Counters, fname, title, parts, srcs, alg_desc, alg_bytes, key, unit):
    """Summary of a unit of work made of several launches: parts = (kernel, grid,
    dispatches per unit)."""
    lines = [f"# {title}", "#", HEAD, "#", c.cal, "#"]
    tot_f = tot_w = 0.0
    for kern, grid, per in parts:
        f, w, fb, wb = c.traffic(kern, grid)
        lines.append(f"# {kern} grid {grid} (KiB/dispatch): FETCH_SIZE " + ", ".join(f"{x:.1f}" for x in f)
                     + "; WRITE_SIZE " + ", ".join(f"{x:.1f}" for x in w))
        tot_f += fb * per
        tot_w += wb * per
        sqo, _ = c.sq_block(ordered(c.smeta, kern, grid), f"{kern} grid {grid}")
        lines += sqo
    lines += [f"# scaled HBM bytes per {unit}: read {tot_f/1e6:.2f} MB + written {tot_w/1e6:.2f} MB = {(tot_f+tot_w)/1e6:.2f} MB",
              f"# algorithmic bytes per {unit}: {alg_desc} = {alg_bytes/1e6:.2f} MB "
              f"(counted / algorithmic = {(tot_f+tot_w)/alg_bytes:.2f})",
              "# The figures below are read by bench.py; source_sha256_16 covers " + ", ".join(srcs) + " (in that order).",
              f"kernel = {' + '.join(p[0] for p in parts)}", f"source_sha256_16 = {sha(srcs)}",
              f"fetch_bytes_per_{unit} = {tot_f:.0f}", f"write_bytes_per_{unit} = {tot_w:.0f}",
              f"{key} = {tot_f + tot_w:.0f}"]
    with open(os.path.join(PROFILES, fname), "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("wrote", fname, f"{(tot_f + tot_w)/1e6:.1f} MB")


def counter_summaries(c: Counters):
    sys.path.insert(0, ROOT)
    import bench
    from workloads import DECODE_PAIR, GLOBAL_PREFILL, STACK, SWA_PREFILL, with_

    def attn_bytes(shape):          # q read, o written, K and V read (bf16)
        q = shape.B * shape.T * shape.Hq * shape.Dh * 2
        kv = 2 * shape.B * shape.T * shape.Hkv * shape.Dh * 2
        return 2 * q + kv

    # the stack's window and global layers: the counter run launches one window
    # layer three times, then one global layer three times
    for nm, shape, pick in (("stack32-window", with_(STACK, W=1024), [0, 1, 2]),
                            ("stack32-global", with_(STACK, W=0), [3, 4, 5])):
        role = nm.split("-")[1]
        write_single(c, f"prefill_attn_final.{nm}.pmc.txt",
                     f"HBM traffic and issue counters of prefill_attn_final (attention | final scan "
                     f"pass) in a {role} layer of stack32-b2-t16512 (B=2, 128 meta + 16384 tokens, 25x64 "
                     f"query heads, 5 KV heads{', window 1024' if shape.W > 0 else ', global'})",
                     "prefill_attn_final", 1914880, pick, FUSED,
                     "attention q, o and prepared K/V (bf16) + the final scan's x, delta, z read and y "
                     "written (2 B each per token-channel) and B, C (2 B per token-state)",
                     attn_bytes(shape) + bench.scan_bytes(shape))
    for nm, shape, grid in (("swa-prefill-b1-t2176", SWA_PREFILL, 223232),
                            ("global-prefill-b4-t8320", GLOBAL_PREFILL, 1925120)):
        write_single(c, f"prefill_attn_final.{nm}.pmc.txt",
                     f"HBM traffic and issue counters of prefill_attn_final (attention | final scan pass) on {nm}",
                     "prefill_attn_final", grid, None, FUSED,
                     "attention q, o and prepared K/V + the final scan's x, delta, z, y and B, C",
                     attn_bytes(shape) + bench.scan_bytes(shape))
    for nm, shape, grid in (("swa-prefill-b1-t2176", SWA_PREFILL, 112640),
                            ("global-prefill-b4-t8320", GLOBAL_PREFILL, 1669120)):
        write_single(c, f"attn_fwd_bf16.{nm}.pmc.txt",
                     f"HBM traffic and issue counters of attn_fwd_bf16 (attention alone over the prepared K/V) on {nm}",
                     "attn_fwd_bf16", grid, None, ATTN,
                     "q and o + rotated K and laid-out V (bf16)", attn_bytes(shape),
                     extra=[f"attention FLOPs per launch {bench.attn_flops(shape):.4g}"])
    write_multi(c, "ssm-branch.swa-prefill-b1-t2176.pmc.txt",
                "HBM traffic of the conv + selective scan branch alone (hm_conv_selective_scan) on "
                "swa-prefill-b1-t2176: aggregate pass, carry pass, final pass (one launch each per call)",
                [("scan_chunk<unsigned short, true, false, true>", 107200, 1), ("scan_carry", 204800, 1),
                 ("scan_chunk<unsigned short, true, true, true>", 108800, 1)], SSM,
                "x, delta, z read and y written (2 B each per token-channel), B and C (2 B per "
                "token-state), A, D and the conv parameters once",
                bench.scan_bytes(SWA_PREFILL), "hbm_bytes_per_call", "call")
    write_multi(c, "step-pair.decode-pair-b64-cache1152.pmc.txt",
                "HBM traffic of one decode step of decode-pair-b64-cache1152 (64 sequences, one token "
                "each, through a producer and a consumer layer sharing a 128 + 1024-row cache; each "
                "layer is one step_fused_bf16 and one step_combine launch)",
                [("step_fused_bf16", 266240, 2), ("step_combine<unsigned short>", 65536, 2)], STEP,
                "both layers read the visible cache rows and read + write their SSM and conv states, "
                "q, x, delta, z, B, C in, out; the producer writes its new K/V row",
                bench.decode_bytes(DECODE_PAIR), "hbm_bytes_per_step", "step")
    m, n, k = 33024, 5440, 1600
    write_multi(c, "linear_bf16_w4.block-stack32-in-proj.pmc.txt",
                "HBM traffic of linear_bf16_w4 on a producer block's in-projection of "
                "block-stack32-b2-t16512 (33024 x 1600 -> 5440 columns split into Q, K, V, x, z)",
                [("linear_bf16_w4", 727040, 1)], LIN,
                "x [33024, 1600] and W [5440, 1600] read once, y [33024, 5440] written (bf16)",
                2.0 * (m * k + n * k + m * n), "hbm_bytes_per_launch", "launch")


def kernel_trace_summary(path, bench_json):
    rows = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            rows[(kname(r["Kernel_Name"]), g, wg)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot = sum(sum(v) for v in rows.values())
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    rl = b["roofline"]
    lines = ["# Kernel durations of the default bench run, per (kernel, launch grid)", "#",
             "# Commands (on the MI355X machine, from /tmp with TMPDIR=/tmp; R = repository root,",
             "# OUT = a scratch directory):",
             "#   " + CMD["kt"], "#   " + CMD["sum"],
             "# Rows: dispatches of bench_kernel_trace.csv grouped by kernel name and grid (threads),",
             "# duration = End_Timestamp - Start_Timestamp.  Workloads by grid:",
             "#   stack32-b2-t16512 (the step): prefill_prep_agg 913280 (18 layers that prepare K/V) or",
             "#     252800 (14 that reuse it), prefill_attn_final 1914880 (29 window + 3 global",
             "#     layers: the window layers' launches are the shorter ones), norm_mean_rows 2113536",
             "#   swa-prefill-b1-t2176: prefill_prep_agg 150720, prefill_attn_final 223232,",
             "#     norm_mean_rows 139264; attn_fwd_bf16 112640 (attention alone); two-stream layer:",
             "#     attn_prep_bf16, attn_fwd_bf16, scan_chunk, scan_carry; cached meta rows: 144320 /",
             "#     204800 / 131072",
             "#   global-prefill-b4-t8320: 915200 / 1925120 / 2129920; attn_fwd_bf16 1669120",
             "#   decode-pair-b64-cache1152: step_fused_bf16 266240, step_combine 65536",
             "#   block and block-stack: rms_norm_rows, linear_bf16(_w4), the mixer's launches",
             "# The at::native rows are torch's own kernels (input generation, the cold-cache flush",
             "# between decode steps, dtype copies); none runs inside a timed region.",
             f"# bench.py's own HIP-event figures in this run: window-layer prefill_attn_final "
             f"{rl['us_per_launch']:.1f} us per launch, global-layer {rl['global']['us_per_launch']:.1f} us "
             f"(roofline.us_per_launch); stack pass {b['ms_per_step']:.3f} ms.",
             "#",
             f"{'kernel':<60} {'grid':>9} {'wg':>4} {'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'%time':>6}"]
    fa = sorted(rows.get(("prefill_attn_final", 1914880, 256), []))
    if fa:
        n = len(fa)
        w, g = fa[: n * 29 // 32], fa[n * 29 // 32:]
        lines.insert(-1, f"# prefill_attn_final 1914880 split: shortest 29/32 of {n} launches (window "
                         f"layers) avg {sum(w)/len(w):.1f} us; longest 3/32 (global) avg {sum(g)/len(g):.1f} us")
    for key, v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{key[0][:60]:<60} {key[1]:>9} {key[2]:>4} {len(v):>6} {sum(v)/len(v):>9.2f} "
                     f"{min(v):>9.2f} {max(v):>9.2f} {100*sum(v)/tot:>6.2f}")
    fname = "stack-kernels.bench-default.kernel-trace.txt"
    with open(os.path.join(PROFILES, fname), "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("wrote", fname)


def main():
    if len(sys.argv) != 2:
        raise SystemExit("usage: python3 bench_profiles.py OUT   (the rocprofv3 output directory)")
    out = sys.argv[1]
    counter_summaries(Counters(out))
    kt = os.path.join(out, "kt", "bench_kernel_trace.csv")
    if os.path.exists(kt):
        kernel_trace_summary(kt, os.path.join(out, "bench_kt.json"))


if __name__ == "__main__":
    main()
