"""The allocation-free decode entry point (hm_mixer_step_noalloc) against
hm_mixer_step: same inputs, bit-identical outputs, states and cache rows, on
two calls in a row (the second with a smaller batch and another position), so
that the static scratch array's leftover contents never leak into a result.
"""
import ctypes

import numpy as np
import pytest

from workloads import DECODE_PAIR, decode_inputs, with_

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import up_inputs  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _pair(shape, seed, noalloc):
    """Producer then consumer of one KV-sharing pair; returns every output."""
    d = decode_inputs(shape, seed)
    t = up_inputs(d, shape.dtype)
    kc, vc = t["k_cache"], t["v_cache"]
    plans = [hm.StepPlan(t[n], kc, vc, shape.n_prev, shape.M, shape.W,
                         rope_base=shape.rope_base, eps=shape.eps, want_branches=True)
             for n in "ab"]
    for p in plans:
        if noalloc:
            # the entry point reads no workspace
            p.args.workspace, p.args.workspace_bytes = None, 0
            st = hm.lib.hm_mixer_step_noalloc(ctypes.byref(p.args), _stream())
            assert st == hm.HM_OK, hm.lib.hm_last_error().decode()
        else:
            p.run()
    torch.cuda.synchronize()
    out = {}
    for n, p in zip("ab", plans):
        out[n + ".out"] = p.out.clone()
        out[n + ".ya"] = p.ya.clone()
        out[n + ".ys"] = p.ys.clone()
        out[n + ".ssm"] = t[n]["ssm_state"].clone()
        out[n + ".conv"] = t[n]["conv_state"].clone()
    out["k_cache"], out["v_cache"] = kc.clone(), vc.clone()
    return out


def test_noalloc_step_matches_the_workspace_entry_point():
    assert hm.lib.hm_mixer_step_noalloc_max_bytes() == 8 << 20
    # first call: the full 64-sequence pair; second: 3 sequences at another
    # position (a smaller input over the scratch the first call filled)
    for shape, seed in ((DECODE_PAIR, 0), (with_(DECODE_PAIR, B=3, n_prev=700), 9)):
        ref = _pair(shape, seed, noalloc=False)
        got = _pair(shape, seed, noalloc=True)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"B={shape.B}: {k} differs"


def test_noalloc_step_rejects_scratch_beyond_the_limit():
    # 1024 sequences need about 13 MB of scratch (8 MiB holds about 640):
    # rejected before any launch, nothing written
    shape = with_(DECODE_PAIR, B=1024)
    dev = "cuda"
    B, Di, Hq, Hkv = shape.B, shape.Di, shape.Hq, shape.Hkv
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=dev)  # noqa: E731
    layer = {"q": z(B, Hq, 64), "k_new": z(B, Hkv, 64), "v_new": z(B, Hkv, 64),
             "x": z(B, Di), "delta": z(B, Di), "Bm": z(B, 16), "Cm": z(B, 16), "z": z(B, Di),
             "conv_state": z(B, Di, 3, dt=torch.float32),
             "ssm_state": z(B, Di, 16, dt=torch.float32),
             "A": z(Di, 16, dt=torch.float32), "D": z(Di, dt=torch.float32),
             "conv_w": z(Di, 4, dt=torch.float32), "conv_b": z(Di, dt=torch.float32),
             "beta_a": z(Di, dt=torch.float32), "beta_s": z(Di, dt=torch.float32)}
    kc = z(B, shape.M + shape.cache_slots, Hkv, 64)
    vc = z(B, shape.M + shape.cache_slots, Hkv, 64)
    p = hm.StepPlan(layer, kc, vc, shape.n_prev, shape.M, shape.W)
    assert hm.lib.hm_mixer_step_workspace(ctypes.byref(p.args)) > 8 << 20
    before = layer["ssm_state"].clone()
    st = hm.lib.hm_mixer_step_noalloc(ctypes.byref(p.args), _stream())
    assert st == hm.HM_ERR_UNSUPPORTED
    assert "8388608" in hm.lib.hm_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(layer["ssm_state"], before)
