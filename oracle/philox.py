"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11, the Philox-4x32
bijection with 10 rounds.  One round maps a 4-word counter (c0, c1, c2, c3)
under a 2-word key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with the 64-bit products split into high/low 32-bit halves; between rounds
the key is advanced by the Weyl increments (W0, W1) modulo 2**32.  The
multipliers and increments are the published ones.

Stream layout used by the Uno sampler (the pages only require independent
uniform draws for the acceptance test and for resampling; this layout is
the reading adopted here): word number ``idx`` of stream ``stream`` under
``seed`` is word ``idx % 4`` of Philox4x32-10 applied to the counter
``(idx//4 mod 2**32, idx//4 >> 32, stream mod 2**32, stream >> 32)`` with key
``(seed mod 2**32, seed >> 32)``.  A word ``w`` becomes the uniform
``(w >> 8) * 2**-24``, an exact dyadic value in [0, 1 - 2**-24].

Everything is vectorised with NumPy uint64 arithmetic: a product of two
32-bit values never exceeds 2**64, so it is exact.
"""

import numpy as np

# Published Philox-4x32 multipliers and Weyl key increments (Salmon et al.).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply the 10-round Philox-4x32 bijection.

    All arguments are integer arrays (or scalars) holding 32-bit values;
    they broadcast against each other.  Returns four uint64 arrays holding
    the 32-bit output words.
    """
    c0, c1, c2, c3, k0, k1 = (np.asarray(v, dtype=np.uint64) & _MASK32
                              for v in (c0, c1, c2, c3, k0, k1))
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    w0 = np.uint64(PHILOX_W0)
    w1 = np.uint64(PHILOX_W1)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + w0) & _MASK32
            k1 = (k1 + w1) & _MASK32
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> _SHIFT32, p0 & _MASK32
        hi1, lo1 = p1 >> _SHIFT32, p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_words(seed, stream, offset, n):
    """Words ``offset .. offset+n-1`` of stream ``stream`` under ``seed``.

    Returns a uint32 array of length ``n``.
    """
    seed = int(seed)
    stream = int(stream)
    idx = np.arange(n, dtype=np.uint64) + np.uint64(int(offset))
    blk = idx >> np.uint64(2)
    lane = (idx & np.uint64(3)).astype(np.int64)
    out = philox4x32_10(
        blk & _MASK32,
        blk >> _SHIFT32,
        np.uint64(stream & 0xFFFFFFFF),
        np.uint64((stream >> 32) & 0xFFFFFFFF),
        np.uint64(seed & 0xFFFFFFFF),
        np.uint64((seed >> 32) & 0xFFFFFFFF),
    )
    words = np.stack(out, axis=-1)  # [n, 4]
    return words[np.arange(n), lane].astype(np.uint32)


def words_to_uniform(words):
    """Map 32-bit words to uniforms ``(w >> 8) * 2**-24`` (float64, exact)."""
    w = np.asarray(words, dtype=np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def philox_uniforms(seed, stream, offset, n):
    """Uniforms in [0, 1 - 2**-24] for words ``offset .. offset+n-1``."""
    return words_to_uniform(philox_words(seed, stream, offset, n))
