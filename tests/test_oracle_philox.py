"""Pins for the oracle's Philox4x32-10 (CPU only).

The oracle's generator is written from Salmon et al. (SC'11).  It is pinned
against rocRAND's independent source-level engine (compiled here for the
host from /opt/rocm/include), word for word, at counters that exercise
every carry of the 128-bit counter and both halves of the key; and against
exact properties of the word-to-uniform map.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def xcheck(tmp_path_factory, repo_root):
    if not os.path.exists(ROCRAND_HEADER) or shutil.which("g++") is None:
        pytest.skip("rocRAND source header or g++ not available")
    out = tmp_path_factory.mktemp("philox") / "philox_xcheck"
    src = os.path.join(repo_root, "tests", "philox_xcheck.cpp")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src,
                    "-o", str(out)], check=True, capture_output=True)

    def run(seed, sub, off, n):
        res = subprocess.run([str(out), str(seed), str(sub), str(off), str(n)],
                             check=True, capture_output=True, text=True)
        return np.array([int(v) for v in res.stdout.split()], dtype=np.uint64)

    return run


CASES = [
    (0, 0, 0, 64),
    (1, 0, 0, 16),
    (0, 1, 0, 16),
    (0xDEADBEEFCAFEF00D, 7, 123, 37),            # both key halves
    (42, 0xFFFFFFFF, 5, 12),                      # stream crosses into its high word below
    (42, 0x1_0000_0003, 9, 12),
    (9, 3, (1 << 34) - 6, 16),                    # block counter crosses 2**32
    (9, 3, (1 << 40) + 3, 8),                     # block index high word non-zero
    (2**64 - 1, 2**64 - 1, 2**64 - 9, 8),          # all-ones key and stream
]


@pytest.mark.parametrize("seed,stream,offset,n", CASES)
def test_words_match_rocrand_source_engine(xcheck, seed, stream, offset, n):
    ref = xcheck(seed, stream, offset, n)
    got = philox.philox_words(seed, stream, offset, n).astype(np.uint64)
    np.testing.assert_array_equal(got, ref)


def test_offset_continuity():
    a = philox.philox_words(5, 2, 0, 103)
    b = np.concatenate([philox.philox_words(5, 2, 0, 41), philox.philox_words(5, 2, 41, 62)])
    np.testing.assert_array_equal(a, b)


def test_streams_and_seeds_differ():
    a = philox.philox_words(0, 0, 0, 256)
    assert not np.array_equal(a, philox.philox_words(0, 1, 0, 256))
    assert not np.array_equal(a, philox.philox_words(1, 0, 0, 256))


def test_uniform_map_endpoints_and_grid():
    w = np.array([0, 255, 256, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    u = philox.words_to_uniform(w)
    assert u[0] == 0.0 and u[1] == 0.0
    assert u[2] == 2.0 ** -24
    assert u[3] == 0.5
    assert u[4] == 1.0 - 2.0 ** -24
    # every value is a multiple of 2**-24 and exactly representable in float32
    uu = philox.philox_uniforms(3, 0, 0, 4096)
    assert np.all(uu * 2 ** 24 == np.floor(uu * 2 ** 24))
    assert np.all(uu.astype(np.float32).astype(np.float64) == uu)
    assert np.all((uu >= 0) & (uu < 1))


def test_uniforms_are_uniform():
    # Kolmogorov-Smirnov distance of 2**16 draws from U[0,1) (crit. ~ 1.63/sqrt(n) at 1%)
    n = 1 << 16
    u = np.sort(philox.philox_uniforms(11, 0, 0, n))
    ecdf_hi = np.arange(1, n + 1) / n
    ecdf_lo = np.arange(0, n) / n
    ks = max(np.max(ecdf_hi - u), np.max(u - ecdf_lo))
    assert ks < 1.63 / np.sqrt(n)
