"""Pins of the cached-meta prefill in the oracle.

The meta tokens are the same constants in front of every sequence, so a
prefill that takes the meta rows' K, V and the SSM-branch states after them
from a cache and computes only the real-token rows must equal the last N rows
of the full prefill over X~ = [meta; tokens] (Hymba blog, "Hymba 的整体架构":
meta tokens prepended to the input).  This splits the whole computation at row
M, so a wrong position offset, visibility index or state hand-off fails it.
"""
import numpy as np
import pytest

import oracle
from workloads import TINY, cached_meta_inputs, with_


@pytest.mark.parametrize("B,M,N,W,Hq,Hkv", [(1, 4, 60, 16, 2, 1), (2, 5, 37, 8, 4, 2),
                                            (3, 16, 20, 0, 2, 2), (1, 3, 2, 4, 2, 1),
                                            (2, 1, 30, 64, 4, 1)])
def test_cached_meta_equals_full_prefill(B, M, N, W, Hq, Hkv):
    shape = with_(TINY, B=B, M=M, N=N, W=W, Hq=Hq, Hkv=Hkv, Di=Hq * TINY.Dh)
    full, tokens, meta = cached_meta_inputs(shape, 7 + M)
    ref = oracle.mixer_prefill(full, M, W, pos0=3)
    cache = oracle.meta_cache(meta)
    got = oracle.mixer_prefill_cached_meta(tokens, cache, M, W, pos0=3)
    for key in ("ya", "ys", "out"):
        np.testing.assert_allclose(got[key], ref[key][:, M:], rtol=1e-11, atol=1e-11,
                                   err_msg=key)
    np.testing.assert_allclose(got["ssm_state"], ref["ssm_state"], rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(got["conv_state"], ref["conv_state"])


def test_meta_cache_states_are_the_scan_of_the_meta_rows():
    """The cached states are those after M steps from zero: continuing the scan
    over the tokens from them equals scanning [meta; tokens] from zero."""
    shape = with_(TINY, B=1, M=6, N=10)
    full, tokens, meta = cached_meta_inputs(shape, 3)
    cache = oracle.meta_cache(meta)
    xc_full, st_full = oracle.causal_conv1d(full["x"], full["conv_w"], full["conv_b"])
    _, h_meta = oracle.selective_scan(xc_full[:, :6], full["delta"][:, :6], full["A"],
                                      full["Bm"][:, :6], full["Cm"][:, :6])
    np.testing.assert_allclose(cache["ssm_state"], h_meta[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(cache["conv_state"],
                                  np.asarray(full["x"][0, 3:6], dtype=np.float64).T)
