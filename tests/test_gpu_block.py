"""GPU parity of whole Hymba blocks and their parts (RMS norm, projection
epilogues, the block, the block stack) against the oracle in float64 on the
same bf16 inputs.  Bar: max |gpu - oracle| <= 2e-2 * max |oracle| per output
tensor; the stack's wiring is checked bit-exactly against the same blocks run
one at a time."""
import numpy as np
import pytest

import oracle
from workloads import (BLOCK_STACK, BLOCK_SWA, block_inputs, block_inputs_torch, bf16_round,
                       stack_layer_roles, with_)

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import assert_close, down, up  # noqa: E402

MATS = ("hidden", "w_in", "w_dbc", "w_out", "w_up", "w_down")

# several 128-row tiles with a ragged tail, meta rows, a window shorter than T
SMALL = with_(BLOCK_SWA, name="block-small", B=2, M=8, N=190, Hq=4, Hkv=2, Di=256, W=64,
              d_model=192, d_ffn=320)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _up(d):
    return {k: up(v, "bf16" if k in MATS else "f32") for k, v in d.items()}


def _oracle_block(shape, inp, hidden, window, kv=None):
    return oracle.block_prefill(hidden, inp, shape.Hq, shape.Hkv, shape.Dh, shape.M, window,
                                kv=kv, rope_base=shape.rope_base, eps=shape.eps)


@pytest.mark.parametrize("rows,width", [(37, 1600), (5, 200), (9, 2056), (6, 100), (1, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rms_norm(rows, width, dtype):
    rng = np.random.default_rng(rows * width)
    x = rng.standard_normal((rows, width)) * 3.0
    if dtype == "bf16":
        x = bf16_round(x)
    else:
        x = x.astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(width)).astype(np.float32)
    got = hm.rms_norm(up(x, dtype), up(w, "f32"), 1e-6)
    torch.cuda.synchronize()
    assert_close(down(got), oracle.rms_norm(x, w, 1e-6), dtype, "rms_norm")


@pytest.mark.parametrize("M,K,segs", [(300, 192, [16, 48, 64]), (2176, 1600, [1600, 16, 16]),
                                      (77, 64, [80]), (4100, 320, [1600, 16, 2384])])
def test_linear_epilogues(M, K, segs):
    """softplus(. + bias) on the first segment, SiLU on the second, an in-place
    residual on the last (the block's step sizes, FFN and skip connections)."""
    rng = np.random.default_rng(M + K + len(segs))
    x = bf16_round(rng.standard_normal((M, K)))
    w = bf16_round(rng.standard_normal((sum(segs), K)) / np.sqrt(K))
    bias = (rng.standard_normal(segs[0]) - 1.0).astype(np.float32)
    res = bf16_round(rng.standard_normal((M, segs[-1])))
    outs = [torch.empty((M, c), dtype=torch.bfloat16, device="cuda") for c in segs]
    r_dev = up(res, "bf16")
    outs[-1] = r_dev                                   # y += x w^T in place
    eps = [{"bias": up(bias, "f32"), "act": "softplus"}]
    if len(segs) > 1:
        eps.append({"act": "silu"})
    eps += [{}] * (len(segs) - len(eps))
    eps[-1] = dict(eps[-1], residual=r_dev)
    got = hm.linear(up(x, "bf16"), up(w, "bf16"), seg_cols=segs, outs=outs, epilogues=eps)
    torch.cuda.synchronize()
    refs = oracle.split_columns(oracle.linear(x, w), segs)
    want = []
    for s, ref in enumerate(refs):
        if s == 0:
            ref = oracle.softplus(ref + bias)
        elif s == 1:
            ref = oracle.silu(ref)
        if s == len(segs) - 1:
            ref = ref + res
        want.append(ref)
    for s, (g, ref) in enumerate(zip(got, want)):
        assert_close(down(g), ref, "bf16", f"segment {s}")


def _block_case(shape, seed, producer, window, kv_np=None):
    inp = block_inputs(shape, seed, 0, producer)
    t = _up(inp)
    hidden = t.pop("hidden")
    h_in = inp["hidden"]
    plan_kv = None
    if kv_np is not None:
        # the producer's K/V, prepared on the GPU by a producer block on the same hidden
        prod = block_inputs(shape, seed + 1, 0, True)
        pt = _up(prod)
        ph = up(h_in, "bf16")
        pt.pop("hidden")
        pp = hm.BlockPlan(pt, ph, shape.Hq, shape.Hkv, shape.M, window, shape.rope_base, shape.eps)
        pp.run()
        plan_kv = pp.kv
    plan = hm.BlockPlan(t, hidden, shape.Hq, shape.Hkv, shape.M, window, shape.rope_base,
                        shape.eps, kv=plan_kv, kv_reuse=plan_kv is not None)
    plan.run()
    torch.cuda.synchronize()
    return inp, h_in, down(hidden)


@pytest.mark.parametrize("window", [64, 0])
def test_block_producer_small(window):
    inp, h_in, got = _block_case(SMALL, 3, True, window)
    ref = _oracle_block(SMALL, inp, h_in, window)
    assert_close(got, ref["hidden"], "bf16", "hidden")
    assert_close(got - h_in, ref["hidden"] - h_in, "bf16", "block increment")


def test_block_consumer_small():
    """A block reusing the K/V that a producer block prepared from the same
    hidden states: the oracle takes the producer's K, V from its own run."""
    shape, window = SMALL, 64
    prod = block_inputs(shape, 5 + 1, 0, True)
    inp, h_in, got = _block_case(shape, 5, False, window, kv_np=True)
    kv = _oracle_block(shape, prod, h_in, window)
    ref = _oracle_block(shape, inp, h_in, window, kv=(kv["k"], kv["v"]))
    assert_close(got, ref["hidden"], "bf16", "hidden")
    assert_close(got - h_in, ref["hidden"] - h_in, "bf16", "block increment")


def test_block_tiny_rows():
    """Degenerate sizes: 3 rows (1 meta + 2 tokens) per sequence, window 1
    (each token sees itself and the meta row), widths of one tile."""
    shape = with_(SMALL, B=2, M=1, N=2, Hq=2, Hkv=1, Di=128, W=1, d_model=64, d_ffn=64)
    inp, h_in, got = _block_case(shape, 9, True, shape.W)
    ref = _oracle_block(shape, inp, h_in, shape.W)
    assert_close(got, ref["hidden"], "bf16", "hidden")
    assert_close(got - h_in, ref["hidden"] - h_in, "bf16", "block increment")


def test_block_swa_full_size():
    """One whole block at the model card's widths (1600, FFN 5504) over the
    swa-prefill rows (1 x (128 + 2048)), every element against the oracle."""
    inp, h_in, got = _block_case(BLOCK_SWA, 0, True, BLOCK_SWA.W)
    ref = _oracle_block(BLOCK_SWA, inp, h_in, BLOCK_SWA.W)
    assert_close(got, ref["hidden"], "bf16", "hidden")
    assert_close(got - h_in, ref["hidden"] - h_in, "bf16", "block increment")


def test_block_stack_small_chain():
    """Four blocks (global, producer, consumer, global): every block against
    the oracle on the GPU's own input to it, and the chained stack bit-exactly
    against those one-at-a-time runs."""
    shape = with_(SMALL, layers=4, global_layers=(0, 3))
    roles = stack_layer_roles(shape)
    assert roles == [(0, 0), (shape.W, 1), (shape.W, 1), (0, 3)]
    layers_np = [block_inputs(shape, 11, l, src == l) for l, (_, src) in enumerate(roles)]
    layers = []
    for d in layers_np:
        t = _up(d)
        t.pop("hidden")
        layers.append(t)
    h0 = layers_np[0]["hidden"]
    hidden = up(h0, "bf16")
    stack = hm.BlockStack(layers, roles, hidden, shape.Hq, shape.Hkv, shape.M, shape.rope_base,
                          shape.eps)
    stack.run()
    torch.cuda.synchronize()
    final = hidden.clone()
    # one block at a time, keeping each block's input
    h = up(h0, "bf16")
    ins, kvs = [], {}
    for l, ((window, src), t) in enumerate(zip(roles, layers)):
        ins.append(down(h))
        p = hm.BlockPlan(t, h, shape.Hq, shape.Hkv, shape.M, window, shape.rope_base, shape.eps,
                         kv=kvs.get(src), kv_reuse=src != l)
        p.run()
        if src == l:
            kvs[l] = p.kv
    torch.cuda.synchronize()
    assert torch.equal(final, h), "stack differs from its blocks run one at a time"
    outs = ins[1:] + [down(h)]
    okv = {}
    for l, (window, src) in enumerate(roles):
        r = _oracle_block(shape, layers_np[l], ins[l], window,
                          kv=None if src == l else okv[src])
        if src == l:
            okv[l] = (r["k"], r["v"])
        assert_close(outs[l], r["hidden"], "bf16", f"block {l}")
        assert_close(outs[l] - ins[l], r["hidden"] - ins[l], "bf16", f"block {l} increment")


def test_block_stack_size_sampled_rows():
    """One producer block at the 32-layer stack's size (2 x (128 + 16384) rows,
    width 1600, FFN 5504) in the launch configuration the benchmark times: it
    equals the composition of the separately checked entry points (RMS norm,
    projections with epilogues, mixer) bit-exactly, and on sampled rows its
    FFN half matches the oracle given the GPU's h1."""
    shape = BLOCK_STACK
    dev = "cuda"
    t = block_inputs_torch(shape, 0, 0, True, dev, hidden=True)
    h_in = t.pop("hidden")
    hidden = h_in.clone()
    plan = hm.BlockPlan(t, hidden, shape.Hq, shape.Hkv, shape.M, shape.W, shape.rope_base,
                        shape.eps)
    plan.run()
    # the same block from its parts
    Qw, KVw, Di = shape.Hq * shape.Dh, shape.Hkv * shape.Dh, shape.Di
    u = hm.rms_norm(h_in, t["ln1"], shape.eps)
    q, k, v, x, z = hm.linear(u, t["w_in"], seg_cols=[Qw, KVw, KVw, Di, Di])
    dt, Bm, Cm = hm.linear(x, t["w_dbc"], seg_cols=[Di, 16, 16],
                           epilogues=[{"bias": t["dt_bias"], "act": "softplus"}, {}, {}])
    B, T = shape.B, shape.T
    mix = {"q": q.view(B, T, shape.Hq, shape.Dh), "k": k.view(B, T, shape.Hkv, shape.Dh),
           "v": v.view(B, T, shape.Hkv, shape.Dh), "x": x, "delta": dt, "Bm": Bm, "Cm": Cm,
           "z": z}
    for key in ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s"):
        mix[key] = t[key]
    mo = hm.mixer_prefill(mix, shape.M, shape.W, rope_base=shape.rope_base, eps=shape.eps,
                          want_states=False)["out"]
    h1 = h_in.clone()
    hm.linear(mo, t["w_out"], outs=[h1], seg_cols=[shape.d_model], epilogues=[{"residual": h1}])
    h2 = h1.clone()
    a = hm.linear(hm.rms_norm(h1, t["ln2"], shape.eps), t["w_up"], epilogues=[{"act": "silu"}],
                  seg_cols=[shape.d_ffn])[0]
    hm.linear(a, t["w_down"], outs=[h2], seg_cols=[shape.d_model], epilogues=[{"residual": h2}])
    torch.cuda.synchronize()
    assert torch.equal(hidden, h2), "block differs from the composition of its parts"
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, shape.M - 1, shape.M, T - 1, 2 * T - 1],
                                     rng.integers(0, B * T, 24)]))
    h1r = down(h1.view(B * T, -1)[torch.as_tensor(rows, device=dev)])
    w = {k2: down(t[k2]) for k2 in ("ln2", "w_up", "w_down")}
    ref = h1r + oracle.ffn(oracle.rms_norm(h1r, w["ln2"], shape.eps), w["w_up"], w["w_down"])
    got = down(hidden.view(B * T, -1)[torch.as_tensor(rows, device=dev)])
    assert_close(got, ref, "bf16", "sampled rows")
    assert_close(got - h1r, ref - h1r, "bf16", "sampled FFN increments")
