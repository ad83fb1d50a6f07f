"""Build libhm.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Usage: python hybrid_head_lm_amd/build.py [--verbose]   (does not import the package)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhm.so")
# the benchmark's instruction-rate probe: its own library, not part of libhm
PROBE_SRC = os.path.join(HERE, "probe", "alu_rate.hip")
PROBE_LIB = os.path.join(HERE, "libhm_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = os.environ.get("HM_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are disabled for every kernel (only scalar fp32 VALU).
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs (no AGPR copies around every MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(HERE, "..", "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Files whose kernels keep MFMA accumulators in AGPRs (more than 256 of them
# per lane): built without the VGPR-only MFMA form.
AGPR_FILES = {"linear_w4.hip"}


def _flags(src: str):
    if os.path.basename(src) in AGPR_FILES:
        return [f for f in CFLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=true")]
    return CFLAGS


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *_flags(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libhm.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile the ALU instruction-rate probe into libhm_probe.so."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
