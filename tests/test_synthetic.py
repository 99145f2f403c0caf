"""Host-side input generators: determinism and bf16 rounding (CPU only)."""

import numpy as np

from synthetic import WORKLOADS, bf16_bits, bf16_round, gate_vector, gemm_inputs, verify_inputs


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -7, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -2.5, 0.0, 3.0e38], dtype=np.float32)
    r = bf16_round(vals)
    np.testing.assert_array_equal(r[:5], np.array([1.0, 1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6,
                                                   1.0 + 2 ** -7], np.float32))
    assert r[5] == -2.5 and r[6] == 0.0
    assert np.all(bf16_bits(r).astype(np.uint32) << 16 == r.view(np.uint32))


def test_gate_layout_is_verify_then_draft_per_sequence():
    g = gate_vector(3, 2, 1)
    np.testing.assert_array_equal(g, [0, 0, 1, 0, 0, 1, 0, 0, 1])
    assert WORKLOADS["layer_b64"].rows == 2048 and WORKLOADS["serve_b256"].rows == 16384


def test_generators_are_seeded():
    a = gemm_inputs(4, 32, 16, 8, seed=5)
    b = gemm_inputs(4, 32, 16, 8, seed=5)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    z1, d1 = verify_inputs(2, 3, 50, seed=9, kind="zipf")
    z2, d2 = verify_inputs(2, 3, 50, seed=9, kind="zipf")
    np.testing.assert_array_equal(z1, z2)
    np.testing.assert_array_equal(d1, d2)
    assert np.all(bf16_round(z1) == z1)
