"""Philox4x64-10 counter-based generator, vectorised over counters (oracle side).

Written from the published definition (J. Salmon, M. Moraes, R. Dror,
D. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): a 4-word
counter and a 2-word key; each of the 10 rounds multiplies words 0 and 2 by
two fixed odd constants, splits each 128-bit product into high and low
halves, and permutes/xors them with words 1 and 3 and the key; between
rounds the key is advanced by two Weyl constants.

The DSpark pages fix no generator; the verifier's draws for request i and
draft position k come from the block at counter (k+1, i, 0, 0) under key
(seed_i, 0).  Word 0 gives the acceptance uniform, word 1 the uniform for
the emitted token.  The draft sampler's draw for the same (i, k) is word 0 of
the block at counter (k+1, i, 1, 0): a separate counter, so one seed can key
both stages without the draft and the acceptance draws coinciding.
Uniforms are 53-bit: (w >> 11) * 2^-53, in [0, 1).

Test infrastructure only (see the package docstring).  Pinned bit for bit
to numpy.random.Philox in tests/test_oracle_philox.py.
"""

import numpy as np

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, b):
    """Full 64x64 -> 128-bit product of uint64 arrays, as (hi, lo)."""
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = (mid << _S32) | (p00 & _LO32)
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """One Philox4x64 block with 10 rounds; all arguments uint64 arrays (broadcast)."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3, k0, k1 = (np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3, k0, k1))
        c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
        c0, c1, c2, c3 = c0.copy(), c1.copy(), c2.copy(), c3.copy()
        k0, k1 = k0.copy(), k1.copy()
        for rnd in range(10):
            if rnd > 0:
                k0 = k0 + _W0
                k1 = k1 + _W1
            hi0, lo0 = _mulhilo(_M0, c0)
            hi1, lo1 = _mulhilo(_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return c0, c1, c2, c3


def to_uniform53(w):
    """53-bit uniform in [0, 1) from a 64-bit word: (w >> 11) * 2^-53 (exact in fp64)."""
    return (np.asarray(w, dtype=np.uint64) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniforms(seed, request, position):
    """(u_accept, u_emit) for request index i and draft position k under key (seed, 0).

    seed: uint64 array-like (per request); request, position: integer arrays,
    broadcast together.  Block counter = (k + 1, i, 0, 0).
    """
    seed = np.asarray(seed, dtype=np.uint64)
    request = np.asarray(request, dtype=np.uint64)
    position = np.asarray(position, dtype=np.uint64)
    w0, w1, _, _ = philox4x64_10(position + np.uint64(1), request, np.uint64(0), np.uint64(0),
                                 seed, np.uint64(0))
    return to_uniform53(w0), to_uniform53(w1)


def draft_uniform(seed, request, position):
    """The draft sampler's uniform for request i and draft position k (0-based): word 0 of the
    block at counter (k + 1, i, 1, 0) under key (seed, 0)."""
    seed = np.asarray(seed, dtype=np.uint64)
    request = np.asarray(request, dtype=np.uint64)
    position = np.asarray(position, dtype=np.uint64)
    w0, _, _, _ = philox4x64_10(position + np.uint64(1), request, np.uint64(1), np.uint64(0),
                                seed, np.uint64(0))
    return to_uniform53(w0)
