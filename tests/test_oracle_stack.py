"""Pins for the glue between projections of the synthetic stack (CPU only)."""

import numpy as np

from oracle import stack


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [-2.0, -2.0]])
    y = stack.rmsnorm(x, eps=0.0 + 1e-300)
    np.testing.assert_allclose(y[0], [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=1e-15)
    np.testing.assert_allclose(y[2], [-1.0, -1.0], rtol=1e-15)
    z = np.random.default_rng(0).standard_normal((4, 64)) * 7
    r = stack.rmsnorm(z, eps=0.0 + 1e-300)
    np.testing.assert_allclose(np.mean(r * r, axis=-1), 1.0, rtol=1e-13)
    # eps enters under the root
    assert abs(stack.rmsnorm(np.array([[1.0]]), eps=3.0)[0, 0] - 0.5) < 1e-15


def test_silu_mul_closed_forms():
    np.testing.assert_allclose(stack.silu_mul([0.0, 1.0, -1.0], [5.0, 2.0, 2.0]),
                               [0.0, 2.0 / (1 + np.exp(-1.0)), -2.0 / (1 + np.exp(1.0))], rtol=1e-15)
    # silu(t) -> t for large t and -> 0 for very negative t
    assert abs(stack.silu_mul([40.0], [1.0])[0] - 40.0) < 1e-12
    assert abs(stack.silu_mul([-40.0], [1.0])[0]) < 1e-15


def test_residual_add():
    np.testing.assert_array_equal(stack.residual_add([1.0, 2.0], [0.5, -2.0]), [1.5, 0.0])
