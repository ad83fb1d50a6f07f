"""The torch binding refuses tensors whose size, rank, dtype or device does
not match the call before anything is launched: the library takes plain pointers
and cannot know a buffer's size, so a short output or parameter tensor would
otherwise be written or read past its end.  No kernel runs in these tests.
"""
import pytest

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _z(*shape, dtype=None):
    return torch.zeros(shape, dtype=dtype or torch.float32, device="cuda")


def test_attention_rejects_mis_sized_tensors():
    q, k = _z(1, 64, 2, 16), _z(1, 64, 1, 16)
    with pytest.raises(ValueError, match="out"):
        hm.swa_meta_attn(q, k, k, 4, 16, out=_z(1, 63, 2, 16))
    with pytest.raises(ValueError, match="out"):
        hm.swa_meta_attn(q, k, k, 4, 16, out=_z(1, 64, 2, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="v"):
        hm.swa_meta_attn(q, k, _z(1, 32, 1, 16), 4, 16)
    with pytest.raises(ValueError, match="dimensions"):
        hm.swa_meta_attn(q[0], k, k, 4, 16)
    with pytest.raises(ValueError, match="device tensors"):
        hm.swa_meta_attn(q, k, k.cpu(), 4, 16)


def test_ssm_branch_rejects_mis_sized_tensors():
    B, T, Di, N = 1, 40, 32, 16
    x, A = _z(B, T, Di), _z(Di, N)
    bc = _z(B, T, N)
    with pytest.raises(ValueError, match="Bm"):
        hm.selective_scan(x, x, A, _z(B, T, 8), bc)
    with pytest.raises(ValueError, match="h_out"):
        hm.selective_scan(x, x, A, bc, bc, h_out=_z(B, Di, 8))
    with pytest.raises(ValueError, match="delta"):
        hm.selective_scan(x, _z(B, T - 1, Di), A, bc, bc)
    with pytest.raises(ValueError, match="conv_state_in"):
        hm.conv_selective_scan(x, _z(Di, 4), _z(Di), x, A, bc, bc, conv_state_in=_z(B, Di, 4))
    with pytest.raises(ValueError, match="w"):
        hm.causal_conv1d(x, _z(Di + 1, 4))
    with pytest.raises(ValueError, match="beta_s"):
        hm.branch_norm_mean(x, x, _z(Di), _z(Di - 1))


def test_projection_rejects_mis_sized_tensors():
    bf = torch.bfloat16
    x, w = _z(8, 64, dtype=bf), _z(48, 64, dtype=bf)
    with pytest.raises(ValueError, match="seg_cols"):
        hm.linear(x, w, seg_cols=[16, 16])
    with pytest.raises(ValueError, match="outs"):
        hm.linear(x, w, seg_cols=[16, 32], outs=[_z(8, 16, dtype=bf), _z(8, 16, dtype=bf)])
    with pytest.raises(ValueError, match="residual"):
        hm.linear(x, w, epilogues=[{"residual": _z(8, 47, dtype=bf)}])
    with pytest.raises(ValueError, match="w"):
        hm.linear(x, _z(48, 32, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        hm.rms_norm(x, _z(64), out=_z(8, 32, dtype=bf))


def test_step_plan_rejects_mis_sized_tensors():
    B, Hq, Hkv, Dh, Di, N, M, W = 2, 2, 1, 16, 32, 16, 4, 16
    layer = {"q": _z(B, Hq, Dh), "x": _z(B, Di), "delta": _z(B, Di), "z": _z(B, Di),
             "Bm": _z(B, N), "Cm": _z(B, N), "conv_state": _z(B, Di, 3),
             "ssm_state": _z(B, Di, N), "A": _z(Di, N), "D": _z(Di), "conv_w": _z(Di, 4),
             "conv_b": _z(Di), "beta_a": _z(Di), "beta_s": _z(Di)}
    kc = _z(B, M + W, Hkv, Dh)
    with pytest.raises(ValueError, match="out"):
        hm.StepPlan(layer, kc, kc, 3, M, W, out=_z(B, Di - 1))
    with pytest.raises(ValueError, match="v_cache"):
        hm.StepPlan(layer, kc, _z(B, M + W - 1, Hkv, Dh), 3, M, W)
    with pytest.raises(ValueError, match="ssm_state"):
        hm.StepPlan(dict(layer, ssm_state=_z(B, Di, 8)), kc, kc, 3, M, W)
    with pytest.raises(ValueError, match="k_new"):
        hm.StepPlan(dict(layer, k_new=_z(B, Hkv, Dh + 1), v_new=_z(B, Hkv, Dh)), kc, kc, 3, M, W)


def test_prefill_and_block_plans_reject_mis_sized_tensors():
    bf = torch.bfloat16
    B, T, Hq, Hkv, Dh, N, M, W = 1, 64, 2, 1, 64, 16, 4, 16
    Di = Hq * Dh
    t = {"q": _z(B, T, Hq, Dh, dtype=bf), "k": _z(B, T, Hkv, Dh, dtype=bf),
         "v": _z(B, T, Hkv, Dh, dtype=bf), "x": _z(B, T, Di, dtype=bf),
         "delta": _z(B, T, Di, dtype=bf), "Bm": _z(B, T, N, dtype=bf), "Cm": _z(B, T, N, dtype=bf),
         "z": _z(B, T, Di, dtype=bf), "A": _z(Di, N), "D": _z(Di), "conv_w": _z(Di, 4),
         "conv_b": _z(Di), "beta_a": _z(Di), "beta_s": _z(Di)}
    with pytest.raises(ValueError, match="z"):
        hm.PrefillPlan(dict(t, z=_z(B, T - 1, Di, dtype=bf)), M, W)
    with pytest.raises(ValueError, match="beta_s"):
        hm.PrefillPlan(dict(t, beta_s=_z(Di + 1)), M, W)
    with pytest.raises(ValueError, match="meta k"):
        hm.PrefillPlan(t, M, W, meta={"k": _z(M + 1, Hkv, Dh, dtype=bf),
                                      "v": _z(M, Hkv, Dh, dtype=bf)})
    with pytest.raises(ValueError, match="out"):
        hm.PrefillPlan(t, M, W, out=_z(B, T, Di - 1, dtype=bf))
    d_model, d_ffn = 128, 192
    w = {"ln1": _z(d_model), "ln2": _z(d_model),
         "w_in": _z(Hq * Dh + 2 * Hkv * Dh + 2 * Di, d_model, dtype=bf),
         "w_dbc": _z(Di + 2 * N, Di, dtype=bf), "dt_bias": _z(Di), "A": _z(Di, N), "D": _z(Di),
         "conv_w": _z(Di, 4), "conv_b": _z(Di), "beta_a": _z(Di), "beta_s": _z(Di),
         "w_out": _z(d_model, Di, dtype=bf), "w_up": _z(d_ffn, d_model, dtype=bf),
         "w_down": _z(d_model, d_ffn, dtype=bf)}
    hidden = _z(B, T, d_model, dtype=bf)
    with pytest.raises(ValueError, match="w_in"):
        # a block that reuses its neighbour's K/V has no K, V rows in w_in
        hm.BlockPlan(w, hidden, Hq, Hkv, M, W, kv=_z(1 << 20, dtype=torch.uint8), kv_reuse=True)
    with pytest.raises(ValueError, match="w_down"):
        hm.BlockPlan(dict(w, w_down=_z(d_model, d_ffn - 64, dtype=bf)), hidden, Hq, Hkv, M, W)
