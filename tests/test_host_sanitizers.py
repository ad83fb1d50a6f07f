"""The library's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Every libhm source is compiled for gfx950 with the sanitizers on its host code
only (-Xarch_host), linked with tests/host/abi_driver.cpp, and the driver runs
every entry point with arguments its validation rejects, plus the size
queries, the status strings and the host-side index function.  Nothing reaches
a kernel launch, so no GPU is needed.  Any sanitizer report or failed
expectation fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_head_lm_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and ROCm clang")
def test_host_layer_under_sanitizers(tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "hybrid_head_lm_amd"))
    import build as hm_build      # the library's own flag set
    objs = []
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(name):
        obj = str(tmp_path / (name[:-4] + ".o"))
        cmd = [HIPCC, *hm_build._flags(os.path.join(CSRC, name)), *SAN_HOST, "-c",
               os.path.join(CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_driver.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                        "-c", os.path.join(ROOT, "tests", "host", "abi_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", drv, *objs,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the library's host code and the driver really are instrumented
    for path in (exe, objs[0]):
        syms = subprocess.run(["nm", path], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, path
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in r.stdout
