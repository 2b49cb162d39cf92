"""The draft sampler's comparison aid (tests/draft_compare.py), on the CPU: elements within the
fp32 accumulation bound of a bf16 rounding boundary get both neighbours; values far from a
boundary get none."""

import numpy as np

from draft_compare import draw_exempt, greedy_ambiguous, rounding_ranges
from oracle.drafting import markov_draft


def _setup():
    V, r = 4, 16
    W1 = np.zeros((V, r))
    W1[0, 0] = 1.0
    W2t = np.zeros((V, r))
    W2t[1, 0] = 2.0 ** -9
    U = np.zeros(V)
    U[1] = 1.0 + 2.0 ** -8 - 2.0 ** -9     # U + b = 1 + 2^-8: exactly a bf16 midpoint
    return U, W1, W2t


def test_midpoint_is_ambiguous():
    U, W1, W2t = _setup()
    out = markov_draft(U[None, None], W1, W2t, [0], temperature=[0.0])
    assert out["logits"][0, 0, 1] == 1.0                     # ties to even
    zlo, zhi, amb = rounding_ranges(U, W1, W2t, 0, "bf16", 2.0 ** -23)
    assert amb.tolist() == [False, True, False, False]
    assert zlo[1] == 1.0 and zhi[1] == 1.0 + 2.0 ** -7
    # no error bound: nothing is ambiguous
    assert not rounding_ranges(U, W1, W2t, 0, "bf16", 0.0)[2].any()


def test_ambiguity_only_where_the_bound_reaches():
    U, W1, W2t = _setup()
    U[1] += 2.0 ** -12                       # 2^-12 away from the midpoint
    assert rounding_ranges(U, W1, W2t, 0, "bf16", 2.0 ** -12)[2][1]
    assert not rounding_ranges(U, W1, W2t, 0, "bf16", 2.0 ** -23)[2].any()


def test_cancellation_near_zero_spans_several_values():
    U, W1, W2t = _setup()
    U[:] = 0.0
    U[1] = -(2.0 ** -9) + 2.0 ** -20
    out = markov_draft(U[None, None], W1, W2t, [0], temperature=[0.0])
    zlo, zhi, amb = rounding_ranges(U, W1, W2t, 0, "bf16", 2.0 ** -12)
    assert amb[1] and zlo[1] < out["logits"][0, 0, 1] < zhi[1]


def test_exemptions():
    z = np.array([0.0, 2.0, 2.0 - 2.0 ** -7, -1.0])
    zlo, zhi = z.copy(), z.copy()
    amb = np.zeros(4, dtype=bool)
    assert not greedy_ambiguous(z, zlo, zhi, amb)
    zhi[2] = 2.0 + 2.0 ** -7                 # element 2 may round above the maximum
    amb[2] = True
    assert greedy_ambiguous(z, zlo, zhi, amb)
    # a draw far from its boundaries is exempt only when the moveable weight reaches the margin
    assert draw_exempt(z, zlo, zhi, amb, 1.0, 1e-3)
    assert not draw_exempt(z, zlo, zhi, np.zeros(4, dtype=bool), 1.0, 1e-3)
    assert draw_exempt(z, zlo, zhi, np.zeros(4, dtype=bool), 1.0, 1e-11)   # the 1e-10 window
