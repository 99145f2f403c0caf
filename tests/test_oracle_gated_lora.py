"""Pins for the oracle's gated-LoRA projection (CPU only).

Against: a hand-derived example (tests/golden/gated_lora_hand.json), a
pure-Python brute-force triple loop on non-square shapes (so a transposed
operand cannot pass), unit-vector probes that read single columns of the
weights back, and the special cases gate = 0 / zero adapter.
"""

import json
import os

import numpy as np
import pytest

from oracle import gated_lora


def test_hand_derived_example(repo_root):
    with open(os.path.join(repo_root, "tests", "golden", "gated_lora_hand.json")) as f:
        g = json.load(f)
    y = gated_lora(np.array(g["x"], float), np.array(g["w"], float), np.array(g["a"], float),
                   np.array(g["b"], float), np.array(g["gate"]), g["scale"])
    np.testing.assert_array_equal(y, np.array(g["y"], float))


def _brute(x, w, a, b, gate, scale):
    M, K = len(x), len(x[0])
    N, r = len(w), len(a)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        t = [sum(x[m][k] * a[j][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            acc = sum(x[m][k] * w[n][k] for k in range(K))
            if gate[m]:
                acc += scale * sum(t[j] * b[n][j] for j in range(r))
            y[m][n] = acc
    return y


@pytest.mark.parametrize("M,K,N,r", [(5, 7, 3, 2), (4, 3, 6, 5), (1, 9, 1, 1), (6, 16, 16, 16)])
def test_brute_force(M, K, N, r):
    rng = np.random.default_rng(M * 1000 + K * 100 + N * 10 + r)
    x, w = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    a, b = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    gate = rng.integers(0, 2, M)
    gate[0] = 1
    ref = np.array(_brute(x.tolist(), w.tolist(), a.tolist(), b.tolist(), gate.tolist(), 2.0))
    got = gated_lora(x, w, a, b, gate, 2.0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_unit_vector_probes():
    rng = np.random.default_rng(7)
    K, N, r = 6, 4, 3
    w, a, b = rng.standard_normal((N, K)), rng.standard_normal((r, K)), rng.standard_normal((N, r))
    eye = np.eye(K)
    y0 = gated_lora(eye, w, a, b, np.zeros(K, np.uint8), 2.0)
    y1 = gated_lora(eye, w, a, b, np.ones(K, np.uint8), 2.0)
    for k in range(K):
        np.testing.assert_allclose(y0[k], w[:, k], rtol=0, atol=1e-15)
        np.testing.assert_allclose(y1[k], w[:, k] + 2.0 * (b @ a[:, k]), rtol=1e-14, atol=1e-14)


def test_gate_zero_rows_are_plain_projection_bitwise():
    rng = np.random.default_rng(3)
    x, w = rng.standard_normal((8, 10)), rng.standard_normal((5, 10))
    a, b = rng.standard_normal((4, 10)), rng.standard_normal((5, 4))
    gate = np.array([0, 1, 0, 1, 1, 0, 0, 1], np.uint8)
    y = gated_lora(x, w, a, b, gate, 2.0)
    plain = gated_lora(x, w, a, b, np.zeros(8, np.uint8), 2.0)
    assert np.array_equal(y[gate == 0], plain[gate == 0])
    zero_adapter = gated_lora(x, w, np.zeros_like(a), b, gate, 2.0)
    np.testing.assert_array_equal(zero_adapter, plain)


def test_rejects_bad_gate_and_shapes():
    x, w = np.ones((2, 3)), np.ones((4, 3))
    a, b = np.ones((1, 3)), np.ones((4, 1))
    with pytest.raises(ValueError):
        gated_lora(x, w, a, b, np.array([0, 2]))
    with pytest.raises(ValueError):
        gated_lora(x, w.T, a, b, np.array([0, 1]))
