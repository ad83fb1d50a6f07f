"""GPU parity of the 32-layer stack at full size (batch 2, 128 + 16384 rows).

Adjacent sliding-window layers share the producer's prepared K/V; layers 0, 15
and 31 are global.  The whole stack runs on the GPU; the oracle then checks
sampled rows of selected layers (global, producer, consumer, unpaired): the
attention rows directly, the SSM branch with a full sequential scan (and the
final conv and SSM states), and the fused output of those rows.
"""
import numpy as np
import pytest

import oracle
from workloads import STACK, prefill_inputs_torch, stack_layer_roles

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import assert_close, down  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_stack_full_size_sampled():
    shape = STACK
    roles = stack_layer_roles(shape)
    dev = torch.device("cuda")
    layers = [prefill_inputs_torch(shape, 0, i, dev) for i in range(shape.layers)]
    stack = hm.StackPlan(layers, roles, shape.M, shape.rope_base, shape.eps, keep_outputs=True)
    stack.run()
    torch.cuda.synchronize()
    rows = np.array([0, 127, 128, 1151, 1152, 5000, 9999, 16383, 16384, 16511])
    # global first, producer, consumer, global middle, unpaired window, global last
    for layer in (0, 1, 2, 15, 30, 31):
        window, src = roles[layer]
        t = layers[layer]
        h = {k: down(v) for k, v in t.items() if k not in ("k", "v")}
        k_src, v_src = down(layers[src]["k"]), down(layers[src]["v"])
        ya_ref = oracle.attention(h["q"], k_src, v_src, shape.M, window, shape.rope_base,
                                  rows=rows).reshape(shape.B, len(rows), shape.Di)
        p = stack.plans[layer]
        assert_close(down(p.ya)[:, rows], ya_ref, "bf16", f"layer {layer} attention rows")
        xc, cs_ref = oracle.causal_conv1d(h["x"], h["conv_w"], h["conv_b"], None, True)
        ys_ref, h_ref = oracle.selective_scan(xc, h["delta"], h["A"], h["Bm"], h["Cm"], h["D"],
                                              h["z"])
        assert_close(down(p.ys)[:, rows], ys_ref[:, rows], "bf16", f"layer {layer} ssm rows")
        assert_close(down(p.h), h_ref, "bf16", f"layer {layer} final state")
        assert np.array_equal(down(p.conv_state), cs_ref), f"layer {layer} conv state"
        out_ref = oracle.branch_norm_mean(ya_ref, ys_ref[:, rows], h["beta_a"], h["beta_s"],
                                          shape.eps)
        assert_close(down(p.out)[:, rows], out_ref, "bf16", f"layer {layer} out rows")
