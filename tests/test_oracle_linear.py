"""Pins of the projection oracle (Hymba blog, "数学表示" §2 and §5)."""
import numpy as np

import oracle


def test_linear_is_the_sum_over_k():
    """Brute force: y[m, n] = sum_k x[m, k] w[n, k]."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = oracle.linear(x, w)
    for m in range(3):
        for n in range(4):
            assert abs(y[m, n] - sum(x[m, k] * w[n, k] for k in range(5))) < 1e-13


def test_linear_batched_and_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 6))
    np.testing.assert_allclose(oracle.linear(x, np.eye(6)), x, rtol=0, atol=0)
    w = rng.standard_normal((4, 6))
    np.testing.assert_allclose(oracle.linear(x, w)[1, 2], w @ x[1, 2], rtol=1e-13)


def test_split_columns():
    y = np.arange(2 * 10).reshape(2, 10)
    a, b, c = oracle.split_columns(y, [3, 5, 2])
    assert a.shape == (2, 3) and b.shape == (2, 5) and c.shape == (2, 2)
    np.testing.assert_array_equal(np.concatenate([a, b, c], axis=1), y)
