"""Pins of the oracle's counter-based generator against numpy's Philox (a library routine)."""

import numpy as np

from oracle.philox import philox4x64_10, to_uniform53, uniforms


def _numpy_block(seed, i, k):
    # numpy advances the counter before producing a block, so counter=[k, i, 0, 0]
    # yields the block at counter (k+1, i, 0, 0).
    # (uint64 arrays: the constructor mis-casts Python ints >= 2^63 given in a list)
    bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                          counter=np.array([k, i, 0, 0], dtype=np.uint64))
    return bg.random_raw(4)


def test_blocks_match_numpy_bit_for_bit():
    rng = np.random.default_rng(7)
    n = 3000
    seeds = rng.integers(0, 2 ** 64, size=n, dtype=np.uint64)
    reqs = rng.integers(0, 2 ** 20, size=n, dtype=np.uint64)
    pos = rng.integers(0, 64, size=n, dtype=np.uint64)
    # extremes of every word
    seeds[:4] = [0, 1, 2 ** 64 - 1, 2 ** 63]
    reqs[:4] = [0, 2 ** 32 - 1, 2 ** 64 - 1, 12345]
    pos[:4] = [0, 63, 2 ** 64 - 2, 1]
    w = philox4x64_10(pos + np.uint64(1), reqs, 0, 0, seeds, 0)
    for t in range(n):
        ref = _numpy_block(seeds[t], reqs[t], pos[t])
        got = [int(w[c][t]) for c in range(4)]
        assert got == [int(x) for x in ref], (t, seeds[t], reqs[t], pos[t])


def test_uniforms_match_numpy_generator_random():
    # numpy's Generator.random() maps a 64-bit word w to (w >> 11) * 2^-53.
    rng = np.random.default_rng(11)
    for _ in range(300):
        s = int(rng.integers(0, 2 ** 64, dtype=np.uint64))
        i = int(rng.integers(0, 4096))
        k = int(rng.integers(0, 32))
        g = np.random.Generator(np.random.Philox(key=np.array([s, 0], dtype=np.uint64),
                                                 counter=np.array([k, i, 0, 0], dtype=np.uint64)))
        ref = g.random(2)
        ua, ue = uniforms(np.uint64(s), i, k)
        assert float(ua) == ref[0] and float(ue) == ref[1]


def test_uniform53_range_and_resolution():
    w = np.array([0, 2 ** 11 - 1, 2 ** 11, 2 ** 64 - 1], dtype=np.uint64)
    u = to_uniform53(w)
    assert u[0] == 0.0 and u[1] == 0.0
    assert u[2] == 2.0 ** -53
    assert u[3] == 1.0 - 2.0 ** -53 and u[3] < 1.0


def test_draft_uniform_matches_numpy_generator():
    # the draft sampler's block is at counter (k+1, i, 1, 0); numpy's counter [k, i, 1, 0]
    # advanced once is that block, and Generator.random() is (w >> 11) * 2^-53 of word 0
    from oracle.philox import draft_uniform
    rng = np.random.default_rng(13)
    for _ in range(300):
        s = int(rng.integers(0, 2 ** 64, dtype=np.uint64))
        i = int(rng.integers(0, 4096))
        k = int(rng.integers(0, 32))
        g = np.random.Generator(np.random.Philox(key=np.array([s, 0], dtype=np.uint64),
                                                 counter=np.array([k, i, 1, 0], dtype=np.uint64)))
        assert float(draft_uniform(np.uint64(s), i, k)) == g.random()
        ua, ue = uniforms(np.uint64(s), i, k)
        assert float(draft_uniform(np.uint64(s), i, k)) not in (float(ua), float(ue))
