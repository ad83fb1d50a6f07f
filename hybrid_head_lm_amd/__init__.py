"""Python binding of libhm, the MI355X (gfx950) hybrid-head mixer core.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/hm.h.  PyTorch provides device
memory (tensors, workspaces) and the current stream.  There is no fallback:
if libhm.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

# torch first: its HIP runtime (soname libamdhip64.so.7) must already be in the
# process when libhm.so is loaded, so that the library binds to that same
# runtime instance (one device context, torch's streams and allocations)
# instead of loading a second copy from /opt/rocm.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhm.so")

HM_OK, HM_ERR_INVALID, HM_ERR_UNSUPPORTED, HM_ERR_WORKSPACE, HM_ERR_HIP = range(5)
HM_F32, HM_BF16 = 0, 1
HM_ACT_NONE, HM_ACT_SILU, HM_ACT_SOFTPLUS = 0, 1, 2

EXPORTS = (
    "hm_abi_version", "hm_status_string", "hm_last_error",
    "hm_swa_meta_attn", "hm_swa_meta_attn_workspace",
    "hm_attn_kv_bytes", "hm_attn_kv_prepare", "hm_attn_with_kv",
    "hm_causal_conv1d", "hm_selective_scan", "hm_selective_scan_workspace",
    "hm_conv_selective_scan", "hm_branch_norm_mean", "hm_linear_bf16", "hm_linear_bf16_ex",
    "hm_rms_norm", "hm_mixer_prefill", "hm_mixer_prefill_workspace",
    "hm_block_prefill", "hm_block_prefill_workspace",
    "hm_mixer_step", "hm_mixer_step_workspace", "hm_mixer_step_noalloc",
    "hm_mixer_step_noalloc_max_bytes",
    "hm_debug_attn_mask", "hm_debug_tile_plan", "hm_debug_attn_tiles", "hm_debug_cache_slot",
    "hm_debug_step_positions",
)


class HmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


_vp = ctypes.c_void_p
_i = ctypes.c_int
_ll = ctypes.c_longlong
_f = ctypes.c_float
_sz = ctypes.c_size_t


class PrefillArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("B", "T", "Hq", "Hkv", "Dh", "Di", "N", "K", "n_meta", "window")] + [
        ("pos0", _ll), ("rope_base", _f), ("scale", _f), ("eps", _f), ("dtype", _i),
    ] + [(n, _vp) for n in ("q", "k", "v", "x", "delta", "Bm", "Cm", "z", "A", "D", "conv_w",
                            "conv_b", "beta_a", "beta_s", "ya", "ys", "out", "conv_state_out",
                            "h_out", "kv")] + [("kv_bytes", _sz), ("kv_reuse", _i),
                                               ("stream2", _vp), ("workspace", _vp),
                                               ("workspace_bytes", _sz)] + [
        (n, _vp) for n in ("meta_k", "meta_v", "conv_state_in", "h0", "events")]


class StepArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("B", "Hq", "Hkv", "Dh", "Di", "N", "K", "n_meta", "window",
                                  "cache_slots")] + [
        ("n_prev", _ll), ("rope_base", _f), ("scale", _f), ("eps", _f), ("dtype", _i),
    ] + [(n, _vp) for n in ("q", "k_new", "v_new", "k_cache", "v_cache", "x", "delta", "Bm", "Cm",
                            "z", "A", "D", "conv_w", "conv_b", "conv_state", "ssm_state",
                            "beta_a", "beta_s", "out", "workspace")] + [
        ("workspace_bytes", _sz), ("ya_out", _vp), ("ys_out", _vp), ("n_prev_seq", _vp)]


class LinearEpilogue(ctypes.Structure):
    _fields_ = [("bias", _vp), ("residual", _vp), ("act", _i)]


class BlockArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("B", "T", "d_model", "d_ffn", "Hq", "Hkv", "Dh", "Di", "N", "K",
                                  "n_meta", "window")] + [
        ("pos0", _ll), ("rope_base", _f), ("scale", _f), ("eps", _f), ("dtype", _i),
    ] + [(n, _vp) for n in ("hidden", "ln1", "ln2", "w_in", "w_dbc", "dt_bias", "A", "D",
                            "conv_w", "conv_b", "beta_a", "beta_s", "w_out", "w_up", "w_down",
                            "kv")] + [("kv_bytes", _sz), ("kv_reuse", _i), ("workspace", _vp),
                                      ("workspace_bytes", _sz)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python hybrid_head_lm_amd/build.py` "
                          "(hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name in EXPORTS:
        getattr(lib, name)      # AttributeError if a declared symbol is missing
    lib.hm_abi_version.restype = _i
    lib.hm_status_string.restype = ctypes.c_char_p
    lib.hm_status_string.argtypes = [_i]
    lib.hm_last_error.restype = ctypes.c_char_p
    lib.hm_swa_meta_attn.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _ll, _f,
                                     _i, _vp, _sz, _vp]
    lib.hm_swa_meta_attn_workspace.argtypes = [_i, _i, _i, _i, _i]
    lib.hm_swa_meta_attn_workspace.restype = _sz
    lib.hm_attn_kv_bytes.argtypes = [_i, _i, _i, _i, _i]
    lib.hm_attn_kv_bytes.restype = _sz
    lib.hm_attn_kv_prepare.argtypes = [_vp, _vp, _vp, _sz, _i, _i, _i, _i, _f, _ll, _i, _vp]
    lib.hm_attn_with_kv.argtypes = [_vp, _vp, _sz, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _ll, _f,
                                    _i, _vp]
    lib.hm_causal_conv1d.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
    lib.hm_selective_scan.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                      _i, _i, _i, _vp, _sz, _vp]
    lib.hm_selective_scan_workspace.argtypes = [_i, _i, _i, _i]
    lib.hm_selective_scan_workspace.restype = _sz
    lib.hm_conv_selective_scan.argtypes = [_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp]
    lib.hm_branch_norm_mean.argtypes = [_vp, _vp, _vp, _vp, _f, _vp, _ll, _i, _i, _vp]
    lib.hm_linear_bf16.argtypes = [_vp, _vp, _i, _i, _i, _i, ctypes.POINTER(_vp),
                                   ctypes.POINTER(_i), _vp]
    lib.hm_linear_bf16_ex.argtypes = [_vp, _vp, _i, _i, _i, _i, ctypes.POINTER(_vp),
                                      ctypes.POINTER(_i), ctypes.POINTER(LinearEpilogue), _vp]
    lib.hm_rms_norm.argtypes = [_vp, _vp, _f, _vp, _ll, _i, _i, _vp]
    lib.hm_block_prefill.argtypes = [ctypes.POINTER(BlockArgs), _vp]
    lib.hm_block_prefill_workspace.argtypes = [ctypes.POINTER(BlockArgs)]
    lib.hm_block_prefill_workspace.restype = _sz
    lib.hm_mixer_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
    lib.hm_mixer_prefill_workspace.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.hm_mixer_prefill_workspace.restype = _sz
    lib.hm_mixer_step.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.hm_mixer_step_workspace.argtypes = [ctypes.POINTER(StepArgs)]
    lib.hm_mixer_step_workspace.restype = _sz
    lib.hm_mixer_step_noalloc.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.hm_mixer_step_noalloc_max_bytes.argtypes = []
    lib.hm_mixer_step_noalloc_max_bytes.restype = _sz
    lib.hm_debug_attn_mask.argtypes = [_i, _i, _i, _vp, _vp]
    lib.hm_debug_tile_plan.argtypes = [_i, _i, _i, _i, _i, _vp, _i, _vp]
    lib.hm_debug_attn_tiles.argtypes = [ctypes.POINTER(_i)] * 3
    lib.hm_debug_attn_tiles.restype = None
    lib.hm_debug_cache_slot.argtypes = [_ll, _i, _i]
    lib.hm_debug_cache_slot.restype = _ll
    lib.hm_debug_step_positions.argtypes = [_i, _ll, _vp, _i, _i, _vp, _vp]
    return lib


lib = _load()
if lib.hm_abi_version() != 1:
    raise ImportError("libhm ABI version mismatch")

from .api import *  # noqa: E402,F401,F403
from .stack import BlockStack, StackPlan  # noqa: E402,F401
