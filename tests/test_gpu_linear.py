"""GPU parity of the projections around the mixer (hm_linear_bf16) against the
oracle's x w^T in float64 on the same bf16 inputs."""
import numpy as np
import pytest

import oracle
from workloads import bf16_round

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("hybrid_head_lm_amd")
torch = pytest.importorskip("torch")
from gpu_util import assert_close, down, up  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# the swa-prefill in-projection (Q, K, V, x, z of 2176 rows from width 1600),
# its out-projection, and small ragged shapes
@pytest.mark.parametrize("M,K,segs", [(2176, 1600, [1600, 320, 320, 1600, 1600]),
                                      (2176, 1600, [1600]), (77, 64, [32, 64]),
                                      (1, 128, [32]), (300, 192, [128, 32, 96]),
                                      (129, 320, [160, 160]),
                                      # 256 x 256 tiles (ragged in both directions)
                                      (4100, 320, [1600, 16, 2384]), (8192, 64, [4096]),
                                      # 192 tiles (the 256 x 256 kernel) and 189 (128 x 128)
                                      (3000, 128, [16, 4080]), (2304, 64, [5376]),
                                      # one tile column, 201 tile rows (last group of the
                                      # grouped tile order holds one row)
                                      (51300, 64, [208])])
def test_linear_bf16(M, K, segs):
    rng = np.random.default_rng(M + K)
    x = bf16_round(rng.standard_normal((M, K)))
    w = bf16_round(rng.standard_normal((sum(segs), K)) / np.sqrt(K))
    outs = hm.linear(up(x, "bf16"), up(w, "bf16"), seg_cols=segs)
    torch.cuda.synchronize()
    refs = oracle.split_columns(oracle.linear(x, w), segs)
    for s, (got, ref) in enumerate(zip(outs, refs)):
        assert got.shape == (M, segs[s])
        assert_close(down(got), ref, "bf16", f"segment {s}")
