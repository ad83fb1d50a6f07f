"""The C-ABI library without a GPU: it loads, exports every symbol include/hm.h
declares, answers its host-side queries, and rejects invalid arguments before
launching anything (these calls never reach a kernel)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hm.h")

hm = pytest.importorskip("hybrid_head_lm_amd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 18
    lib = ctypes.CDLL(hm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(hm.EXPORTS) | {"hm_abi_version"}


def test_version_and_status_strings():
    assert hm.lib.hm_abi_version() == 1
    for code, name in enumerate(["HM_OK", "HM_ERR_INVALID", "HM_ERR_UNSUPPORTED",
                                 "HM_ERR_WORKSPACE", "HM_ERR_HIP"]):
        assert hm.lib.hm_status_string(code).decode() == name


def test_cache_slot_matches_oracle():
    for n_prev in (0, 1, 5, 1023, 1024, 2048, 99999):
        for M, W in ((128, 1024), (4, 16), (0, 1), (3, 0)):
            assert hm.debug_cache_slot(n_prev, M, W) == oracle.cache_slot(n_prev, M, W)
    assert hm.debug_cache_slot(-1, 1, 1) == -1


def test_step_key_splits_fit_the_combine():
    """A global layer's decode at one sequence and a long cache: the key splits
    are capped so that every (query head, split) fits the combine (at most 2048
    of them), which the workspace size shows (one partial of Dh + 2 floats
    per split, KV head and query head of the group)."""
    L = hm.lib
    for n_prev in (3000, 6000, 10240, 16384):
        a = hm.StepArgs(B=1, Hq=25, Hkv=5, Dh=64, Di=1600, N=16, K=4, n_meta=128, window=0,
                        cache_slots=16512, n_prev=n_prev, dtype=hm.HM_BF16)
        nb = L.hm_mixer_step_workspace(ctypes.byref(a))
        ys = -(-1600 // 64) * 64 * 4
        part_floats = (nb - ys) // 4
        n_split = part_floats // (5 * 5 * 66)
        assert 1 <= n_split and 25 * n_split <= 2048, (n_prev, n_split)
        # and the splits cover every visible tile
        tiles = -(-(128 + n_prev + 1) // 64)
        assert n_split * -(-tiles // n_split) >= tiles


def test_workspace_queries():
    L = hm.lib
    assert L.hm_swa_meta_attn_workspace(1, 2176, 5, 64, hm.HM_BF16) == 2 * 5 * 2176 * 64 * 2
    assert L.hm_swa_meta_attn_workspace(1, 64, 1, 16, hm.HM_F32) == 2 * 64 * 16 * 4
    assert L.hm_attn_kv_bytes(1, 2176, 5, 64, hm.HM_BF16) == 2 * 5 * 2176 * 64 * 2
    assert L.hm_swa_meta_attn_workspace(0, 64, 1, 16, hm.HM_F32) == 0
    assert L.hm_selective_scan_workspace(1, 2176, 1600, 16) > 0
    assert L.hm_selective_scan_workspace(1, 2176, 1600, 8) == 0
    a = hm.StepArgs(B=64, Hq=25, Hkv=5, Dh=64, Di=1600, N=16, K=4, n_meta=128, window=1024,
                    cache_slots=1024, n_prev=2048, dtype=hm.HM_BF16)
    nb = L.hm_mixer_step_workspace(ctypes.byref(a))
    # SSM branch output + at least one (max, sum, O) partial per (sequence, head)
    assert nb >= 64 * 1600 * 4 + 64 * 25 * 66 * 4
    a.dtype = hm.HM_F32
    assert L.hm_mixer_step_workspace(ctypes.byref(a)) >= 64 * 1600 * 4 + 64 * 25 * 66 * 4


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: every call below fails validation


def _err():
    return hm.lib.hm_last_error().decode()


def test_attention_rejects_bad_arguments():
    L = hm.lib
    q, k, v, o, ws = (ctypes.c_void_p(i << 20) for i in range(1, 6))
    args = [q, k, v, o, 1, 64, 2, 1, 16, 4, 16, 1e4, 0, 0.0, hm.HM_F32, ws, 1 << 30, None]
    bad = list(args); bad[0] = None
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_INVALID and "q" in _err()
    bad = list(args); bad[7] = 3                      # Hq % Hkv != 0 (Hq=2, Hkv=3)
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_INVALID
    bad = list(args); bad[9] = 65                     # n_meta > T
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_INVALID
    bad = list(args); bad[8] = 48                     # f32 head dim 48
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_UNSUPPORTED
    bad = list(args); bad[14] = hm.HM_BF16            # bf16 needs Dh = 64
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_UNSUPPORTED
    bad = list(args); bad[16] = 16                    # short workspace
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_WORKSPACE
    bad = list(args); bad[3] = q                      # o aliases q
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_INVALID
    bad = list(args); bad[1] = ctypes.c_void_p((1 << 20) + 4)   # misaligned k
    assert L.hm_swa_meta_attn(*bad) == hm.HM_ERR_INVALID


def test_scan_and_conv_reject_bad_arguments():
    L = hm.lib
    y = ctypes.c_void_p(3 << 20)
    assert L.hm_selective_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, y, None,
                               1, 64, 32, 8, hm.HM_F32, FAKE, 1 << 30, None) == hm.HM_ERR_UNSUPPORTED
    assert L.hm_selective_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, y, None,
                               1, 0, 32, 16, hm.HM_F32, FAKE, 1 << 30, None) == hm.HM_ERR_INVALID
    assert L.hm_selective_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, y, None,
                               1, 64, 32, 16, hm.HM_F32, FAKE, 4, None) == hm.HM_ERR_WORKSPACE
    assert L.hm_selective_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                               1, 64, 32, 16, hm.HM_F32, FAKE, 1 << 30, None) == hm.HM_ERR_INVALID
    assert L.hm_causal_conv1d(FAKE, FAKE, None, None, y, None, 1, 8, 4, 3, 1, hm.HM_F32,
                              None) == hm.HM_ERR_UNSUPPORTED
    assert L.hm_causal_conv1d(None, FAKE, None, None, y, None, 1, 8, 4, 4, 1, hm.HM_F32,
                              None) == hm.HM_ERR_INVALID
    assert L.hm_branch_norm_mean(FAKE, FAKE, FAKE, FAKE, -1.0, y, 4, 8, hm.HM_F32,
                                 None) == hm.HM_ERR_INVALID
    assert L.hm_branch_norm_mean(FAKE, FAKE, FAKE, FAKE, 1e-6, y, 4, 8, 7, None) == hm.HM_ERR_UNSUPPORTED


def test_step_and_prefill_reject_bad_arguments():
    L = hm.lib
    a = hm.StepArgs(B=2, Hq=2, Hkv=1, Dh=16, Di=32, N=16, K=4, n_meta=4, window=16,
                    cache_slots=8, n_prev=3, rope_base=1e4, eps=1e-6, dtype=hm.HM_F32)
    assert L.hm_mixer_step(ctypes.byref(a), None) == hm.HM_ERR_INVALID      # slots < window
    a.cache_slots = 16
    a.Di = 31
    assert L.hm_mixer_step(ctypes.byref(a), None) == hm.HM_ERR_INVALID      # Di != Hq*Dh
    a.Di = 32
    a.N = 8
    assert L.hm_mixer_step(ctypes.byref(a), None) == hm.HM_ERR_UNSUPPORTED
    a.N = 16
    assert L.hm_mixer_step(ctypes.byref(a), None) == hm.HM_ERR_INVALID      # NULL pointers
    p = hm.PrefillArgs(B=1, T=64, Hq=2, Hkv=1, Dh=16, Di=32, N=16, K=4, n_meta=4, window=16,
                       rope_base=1e4, eps=1e-6, dtype=hm.HM_F32)
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_INVALID   # NULL outputs
    assert L.hm_mixer_prefill(None, None) == hm.HM_ERR_INVALID


def test_prefill_cached_meta_rejects_unsupported_modes():
    """Cached meta tokens run only on the fused bf16 path: f32, a second
    stream or a missing meta_v are refused before anything is launched."""
    L = hm.lib
    p = hm.PrefillArgs(B=1, T=64, Hq=2, Hkv=1, Dh=64, Di=128, N=16, K=4, n_meta=4, window=16,
                       rope_base=1e4, eps=1e-6, dtype=hm.HM_BF16)
    for i, name in enumerate(("ya", "ys", "out")):
        setattr(p, name, FAKE.value + 4096 * i)
    p.meta_k = FAKE
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_INVALID   # meta_v missing
    p.meta_v = FAKE
    p.n_meta = 0
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_INVALID   # no meta rows
    p.n_meta = 4
    p.dtype = hm.HM_F32
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_UNSUPPORTED
    p.dtype = hm.HM_BF16
    p.stream2 = FAKE
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_UNSUPPORTED
    # the prepared K/V covers the meta rows too
    p.stream2 = None
    n_plain = L.hm_mixer_prefill_workspace(ctypes.byref(p))
    assert n_plain >= L.hm_attn_kv_bytes(1, 68, 1, 64, hm.HM_BF16)


def test_ctypes_structs_match_the_header(tmp_path):
    """The binding's argument-struct layouts equal the C ones."""
    import shutil
    import subprocess
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    pairs = [(hm.PrefillArgs, "hm_prefill_args"), (hm.StepArgs, "hm_step_args"),
             (hm.BlockArgs, "hm_block_args"), (hm.LinearEpilogue, "hm_linear_epilogue")]
    src = tmp_path / "sz.cpp"
    lines = ['#include "hm.h"', "#include <cstdio>", "#include <cstddef>", "int main() {"]
    for cls, cname in pairs:
        lines.append(f'printf("%zu\\n", sizeof({cname}));')
        lines += [f'printf("%zu\\n", offsetof({cname}, {f}));' for f, _ in cls._fields_]
    lines += ["return 0; }"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "sz"
    subprocess.run([cxx, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in
            subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    for cls, cname in pairs:
        n = len(cls._fields_)
        assert vals[0] == ctypes.sizeof(cls), cname
        assert vals[1:1 + n] == [getattr(cls, f).offset for f, _ in cls._fields_], cname
        vals = vals[1 + n:]
    assert vals == []


# The decode-step argument struct as the contract fixes it (field order and
# types); the library's hm_step_args must start with exactly this prefix, so a
# caller built against the contract passes every field where the library
# reads it.  Optional fields may only follow workspace_bytes.
STEP_CONTRACT = """
typedef struct {
  int B, Hq, Hkv, Dh, Di, N, K, n_meta, window, cache_slots; long long n_prev;
  float rope_base, scale, eps; hm_dtype dtype;
  const void *q, *k_new, *v_new;
  void *k_cache, *v_cache;
  const void *x, *delta, *Bm, *Cm, *z;
  const float *A, *D, *conv_w, *conv_b;
  float *conv_state, *ssm_state;
  const float *beta_a, *beta_s;
  void *out;
  void *workspace; size_t workspace_bytes;
} step_contract;
"""
STEP_CONTRACT_FIELDS = ("B", "Hq", "Hkv", "Dh", "Di", "N", "K", "n_meta", "window",
                        "cache_slots", "n_prev", "rope_base", "scale", "eps", "dtype", "q",
                        "k_new", "v_new", "k_cache", "v_cache", "x", "delta", "Bm", "Cm", "z",
                        "A", "D", "conv_w", "conv_b", "conv_state", "ssm_state", "beta_a",
                        "beta_s", "out", "workspace", "workspace_bytes")


def test_step_args_start_with_the_contract_prefix(tmp_path):
    import shutil
    import subprocess
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "contract.cpp"
    lines = ['#include "hm.h"', "#include <cstdio>", "#include <cstddef>", STEP_CONTRACT,
             "int main() {"]
    for f in STEP_CONTRACT_FIELDS:
        lines.append(f'printf("%zu %zu\\n", offsetof(step_contract, {f}), '
                     f'offsetof(hm_step_args, {f}));')
    lines += ['printf("%zu %zu\\n", sizeof(step_contract), offsetof(hm_step_args, ya_out));',
              "return 0; }"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "contract"
    subprocess.run([cxx, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    rows = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    pairs = [tuple(int(v) for v in r.split()) for r in rows if r.strip()]
    assert len(pairs) == len(STEP_CONTRACT_FIELDS) + 1
    for f, (want, got) in zip(STEP_CONTRACT_FIELDS, pairs):
        assert want == got, f"hm_step_args.{f} at offset {got}, the contract puts it at {want}"
        assert getattr(hm.StepArgs, f).offset == want, f
    # the optional fields start where the contract's struct ends
    assert pairs[-1][0] <= pairs[-1][1]


def test_empty_extents_are_rejected():
    """Zero batch, rows or width: HM_ERR_INVALID from every entry point, with
    nothing launched (the pointers are never dereferenced)."""
    L = hm.lib
    q, k, v, o, ws = (ctypes.c_void_p(i << 20) for i in range(1, 6))
    for B, T in ((0, 64), (1, 0)):
        assert L.hm_swa_meta_attn(q, k, v, o, B, T, 2, 1, 16, 0, 16, 1e4, 0, 0.0, hm.HM_F32, ws,
                                  1 << 30, None) == hm.HM_ERR_INVALID
        assert L.hm_causal_conv1d(q, k, None, None, o, None, B, T, 4, 4, 1, hm.HM_F32,
                                  None) == hm.HM_ERR_INVALID
        assert L.hm_conv_selective_scan(q, k, None, None, None, v, FAKE, FAKE, FAKE, None, None,
                                        None, o, None, B, T, 32, 4, 16, hm.HM_F32, ws, 1 << 30,
                                        None) == hm.HM_ERR_INVALID
    assert L.hm_branch_norm_mean(q, k, v, FAKE, 1e-6, o, 0, 8, hm.HM_F32,
                                 None) == hm.HM_ERR_INVALID
    assert L.hm_branch_norm_mean(q, k, v, FAKE, 1e-6, o, 4, 0, hm.HM_F32,
                                 None) == hm.HM_ERR_INVALID
    p = hm.PrefillArgs(B=1, T=0, Hq=2, Hkv=1, Dh=16, Di=32, N=16, K=4, n_meta=0, window=16,
                       rope_base=1e4, eps=1e-6, dtype=hm.HM_F32)
    p.ya, p.ys, p.out = q.value, k.value, v.value
    p.workspace, p.workspace_bytes = ws.value, 1 << 30
    assert L.hm_mixer_prefill(ctypes.byref(p), None) == hm.HM_ERR_INVALID
    s = hm.StepArgs(B=0, Hq=2, Hkv=1, Dh=16, Di=32, N=16, K=4, n_meta=4, window=16,
                    cache_slots=16, n_prev=3, rope_base=1e4, eps=1e-6, dtype=hm.HM_F32)
    assert L.hm_mixer_step(ctypes.byref(s), None) == hm.HM_ERR_INVALID


def test_linear_rejects_bad_arguments():
    L = hm.lib
    outs = (ctypes.c_void_p * 2)(3 << 20, 4 << 20)
    widths = (ctypes.c_int * 2)(32, 64)
    x, w = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20)
    assert L.hm_linear_bf16(x, w, 8, 96, 100, 2, outs, widths, None) == hm.HM_ERR_UNSUPPORTED
    assert L.hm_linear_bf16(x, w, 8, 95, 64, 2, outs, widths, None) == hm.HM_ERR_INVALID
    bad = (ctypes.c_int * 2)(40, 56)                  # not multiples of 16
    assert L.hm_linear_bf16(x, w, 8, 96, 64, 2, outs, bad, None) == hm.HM_ERR_INVALID
    assert L.hm_linear_bf16(x, w, 0, 96, 64, 2, outs, widths, None) == hm.HM_ERR_INVALID
    assert L.hm_linear_bf16(x, w, 8, 96, 64, 9, outs, widths, None) == hm.HM_ERR_INVALID
    alias = (ctypes.c_void_p * 2)(1 << 20, 4 << 20)   # output aliases x
    assert L.hm_linear_bf16(x, w, 8, 96, 64, 2, alias, widths, None) == hm.HM_ERR_INVALID


def test_linear_epilogues_reject_bad_arguments():
    L = hm.lib
    outs = (ctypes.c_void_p * 2)(3 << 20, 4 << 20)
    widths = (ctypes.c_int * 2)(16, 80)
    x, w = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20)
    ep = (hm.LinearEpilogue * 2)()
    ep[0].act = 7                                      # unknown activation
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, outs, widths, ep, None) == hm.HM_ERR_INVALID
    ep[0].act = hm.HM_ACT_SILU
    ep[1].residual = 3 << 20                           # another segment's output
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, outs, widths, ep, None) == hm.HM_ERR_INVALID
    ep[1].residual = 1 << 20                           # x
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, outs, widths, ep, None) == hm.HM_ERR_INVALID
    ep[1].residual = None
    ep[0].bias = (1 << 20) + 4                         # misaligned bias
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, outs, widths, ep, None) == hm.HM_ERR_INVALID
    ep[0].bias = None
    ep[1].residual = (4 << 20) + 8                     # misaligned residual
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, outs, widths, ep, None) == hm.HM_ERR_INVALID
    same = (ctypes.c_void_p * 2)(3 << 20, 3 << 20)     # two segments, one tensor
    assert L.hm_linear_bf16_ex(x, w, 8, 96, 64, 2, same, widths, None, None) == hm.HM_ERR_INVALID


def test_rms_norm_rejects_bad_arguments():
    L = hm.lib
    x, wv, o = (ctypes.c_void_p(i << 20) for i in range(1, 4))
    assert L.hm_rms_norm(x, wv, 1e-6, o, 0, 64, hm.HM_BF16, None) == hm.HM_ERR_INVALID
    assert L.hm_rms_norm(x, wv, 1e-6, o, 4, 0, hm.HM_BF16, None) == hm.HM_ERR_INVALID
    assert L.hm_rms_norm(x, wv, -1.0, o, 4, 64, hm.HM_BF16, None) == hm.HM_ERR_INVALID
    assert L.hm_rms_norm(x, wv, 1e-6, x, 4, 64, hm.HM_BF16, None) == hm.HM_ERR_INVALID
    assert L.hm_rms_norm(x, wv, 1e-6, o, 4, 64, 5, None) == hm.HM_ERR_UNSUPPORTED


def _block_args(**kw):
    a = hm.BlockArgs(B=1, T=200, d_model=192, d_ffn=320, Hq=4, Hkv=2, Dh=64, Di=256, N=16, K=4,
                     n_meta=8, window=64, rope_base=1e4, eps=1e-6, dtype=hm.HM_BF16)
    for f in ("hidden", "ln1", "ln2", "w_in", "w_dbc", "dt_bias", "A", "D", "conv_w", "conv_b",
              "beta_a", "beta_s", "w_out", "w_up", "w_down"):
        setattr(a, f, FAKE.value)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_block_workspace_and_rejections():
    L = hm.lib
    a = _block_args()
    nb = L.hm_block_prefill_workspace(ctypes.byref(a))
    R = 200
    # at least the block's own tensors (norm output, Q, K, V, x, z, step sizes, B, C,
    # both branch outputs, the mixer output) and the prepared K/V held in the workspace
    assert nb >= R * 2 * (192 + 256 + 2 * 128 + 256 * 3 + 2 * 16 + 3 * 256) + 2 * 2 * 256 * 64 * 2
    a.workspace, a.workspace_bytes = 5 << 20, nb
    cases = [
        (dict(dtype=hm.HM_F32), hm.HM_ERR_UNSUPPORTED),
        (dict(d_ffn=330), hm.HM_ERR_UNSUPPORTED),
        (dict(d_model=100), hm.HM_ERR_UNSUPPORTED),
        (dict(Dh=32, Di=128), hm.HM_ERR_UNSUPPORTED),
        (dict(Di=200), hm.HM_ERR_INVALID),
        (dict(T=0), hm.HM_ERR_INVALID),
        (dict(B=0), hm.HM_ERR_INVALID),
        (dict(kv_reuse=1), hm.HM_ERR_INVALID),
        (dict(w_up=None), hm.HM_ERR_INVALID),
        (dict(ln2=(1 << 20) + 4), hm.HM_ERR_INVALID),
        (dict(workspace_bytes=nb - 256), hm.HM_ERR_WORKSPACE),
        (dict(workspace=None), hm.HM_ERR_WORKSPACE),
    ]
    for kw, want in cases:
        b = _block_args(workspace=5 << 20, workspace_bytes=nb)
        for k, v in kw.items():
            setattr(b, k, v)
        assert L.hm_block_prefill(ctypes.byref(b), None) == want, (kw, _err())
    assert L.hm_block_prefill(None, None) == hm.HM_ERR_INVALID
    assert L.hm_block_prefill_workspace(ctypes.byref(_block_args(T=0))) == 0
