"""GPU Philox uniforms vs the oracle's independent implementation: bit-exact."""

import numpy as np
import pytest

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_host

CASES = [
    (0, 0, 0, 1),
    (0, 0, 0, 4097),
    (7, 1, 3, 1000),                       # offset not a multiple of 4
    (2 ** 40 + 5, 2 ** 33 + 1, 2 ** 36 + 2, 777),
    (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 100, 100),   # ends exactly at 2^64
    (123, 0, (1 << 34) - 7, 50),           # block counter crosses 2^32
]


@pytest.mark.gpu
@pytest.mark.parametrize("seed,stream,offset,n", CASES)
def test_philox_bit_exact(seed, stream, offset, n):
    say(f"philox seed={seed} stream={stream} offset={offset} n={n}")
    got = to_host(uno.philox_uniforms(seed, stream, offset, n)).astype(np.float64)
    ref = oracle.philox_uniforms(seed, stream, offset, n)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.gpu
def test_philox_offset_continuity_and_empty():
    say("philox continuity")
    a = to_host(uno.philox_uniforms(9, 2, 5, 3001))
    b = np.concatenate([to_host(uno.philox_uniforms(9, 2, 5, 1234)), to_host(uno.philox_uniforms(9, 2, 1239, 1767))])
    np.testing.assert_array_equal(a, b)
    assert uno.philox_uniforms(9, 2, 5, 0).numel() == 0
