"""Pins of the left-to-right verification oracle (`oracle.verify_left_to_right`).

DSpark paper, §2.1: verification proceeds left to right and the first rejection discards every
later draft token.  The walk is pinned to

* the vectorised `oracle.verify` (itself pinned by the chi-square, closed-form and worked-example
  tests of test_oracle_verify.py) on valid data: the same accepted lengths, tokens, flags and
  draw counts, and the same acceptance ratios up to the first rejection;
* the invariance that defines it: nothing after the first rejection is read, so rewriting those
  rows (NaN, +inf, other values) changes no output;
* its status rule: a bad row at or before the first rejection, or a bad appended-token row when
  every draft passed, is reported; the argument checks stay up front.
"""

import numpy as np
import pytest

import oracle


def _batch(seed, B=32, G=5, V=40, greedy_every=5, topk_every=4):
    rng = np.random.default_rng(seed)
    target = rng.normal(0, 2.0, (B, G + 1, V))
    draft = target[:, :G] + rng.normal(0, 0.7, (B, G, V))
    tokens = np.empty((B, G), dtype=np.int64)
    for i in range(B):
        for k in range(G):
            p = np.exp(draft[i, k] - draft[i, k].max())
            tokens[i, k] = rng.choice(V, p=p / p.sum())
    lengths = rng.integers(0, G + 1, B)
    T = rng.uniform(0.6, 1.3, B)
    T[::greedy_every] = 0.0
    K = np.zeros(B, dtype=np.int64)
    K[1::topk_every] = 7
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    return target, draft, tokens, lengths, T, K, seeds


def _both(args):
    a = oracle.verify(*args)
    b = oracle.verify_left_to_right(*args)
    return a, b


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_walk_equals_vectorised_on_valid_data(seed):
    args = _batch(seed)
    a, b = _both(args)
    for key in ("num_accepted", "out_tokens", "status", "accept_flags", "emit_flag", "draws"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    n, L = a["num_accepted"], args[3]
    G = args[2].shape[1]
    for i in range(len(n)):
        upto = min(int(n[i]) + 1, int(L[i]))   # the positions the walk tested
        np.testing.assert_array_equal(a["accept_prob"][i, :upto], b["accept_prob"][i, :upto])
        assert np.isnan(b["accept_prob"][i, upto:G]).all()
    # the batch exercises rejections, full acceptance, greedy rows and L = 0
    assert (n < L).any() and (n == L).any() and (L == 0).any()


def test_rows_after_the_first_rejection_are_never_read():
    target, draft, tokens, lengths, T, K, seeds = _batch(21, B=48)
    base = oracle.verify_left_to_right(target, draft, tokens, lengths, T, K, seeds)
    n = base["num_accepted"]
    rejected = np.nonzero(n < lengths)[0]
    assert len(rejected) > 10
    rng = np.random.default_rng(5)
    for fill in (np.nan, np.inf, None):
        t2, d2 = target.copy(), draft.copy()
        for i in rejected:
            j = int(n[i])
            if fill is None:
                t2[i, j + 1:] = rng.normal(0, 5.0, t2[i, j + 1:].shape)
                d2[i, j + 1:] = rng.normal(0, 5.0, d2[i, j + 1:].shape)
            else:
                t2[i, j + 1:] = fill
                d2[i, j + 1:] = fill
        out = oracle.verify_left_to_right(t2, d2, tokens, lengths, T, K, seeds)
        for key in base:
            np.testing.assert_array_equal(base[key], out[key], err_msg=f"{key} fill={fill}")
    # the vectorised verify reads every row and reports them
    t2 = target.copy()
    i = int(rejected[0])
    t2[i, int(n[i]) + 1, 0] = np.nan
    if int(n[i]) + 1 <= int(lengths[i]):
        assert oracle.verify(t2, draft, tokens, lengths, T, K, seeds)["status"][i] == oracle.STATUS_NONFINITE


def test_bad_rows_the_walk_reaches():
    target, draft, tokens, lengths, T, K, seeds = _batch(31, B=48)
    base = oracle.verify_left_to_right(target, draft, tokens, lengths, T, K, seeds)
    n = base["num_accepted"]
    seen = set()
    for i in range(len(n)):
        L, ni = int(lengths[i]), int(n[i])
        cases = [("target", j) for j in range(ni + 1)]              # rows 0 .. n (row L when all pass)
        if T[i] != 0.0:
            cases += [("draft", j) for j in range(min(ni + 1, L))]  # draft rows the tests read
        for which, j in cases:
            t2, d2 = target.copy(), draft.copy()
            (t2 if which == "target" else d2)[i, j, 3] = np.nan
            out = oracle.verify_left_to_right(t2, d2, tokens, lengths, T, K, seeds)
            assert out["status"][i] == oracle.STATUS_NONFINITE, (i, which, j)
            assert out["num_accepted"][i] == 0 and (out["out_tokens"][i] == -1).all()
            assert np.isnan(out["accept_prob"][i]).all()
            others = np.arange(len(n)) != i
            np.testing.assert_array_equal(out["num_accepted"][others], n[others])
            seen.add((which, j == ni, ni == L))
    # a bad row before the rejection, at it, and the appended-token row were all exercised
    assert ("target", True, True) in seen and ("target", True, False) in seen and ("draft", True, False) in seen


def test_argument_checks_stay_up_front():
    target, draft, tokens, lengths, T, K, seeds = _batch(41, B=8, greedy_every=100)
    lengths = np.full(8, 4)
    base = oracle.verify_left_to_right(target, draft, tokens, lengths, T, K, seeds)
    i = int(np.argmin(base["num_accepted"]))
    tok2 = tokens.copy()
    tok2[i, 3] = 10_000                       # a bad token at the last position, past any rejection
    out = oracle.verify_left_to_right(target, draft, tok2, lengths, T, K, seeds)
    assert out["status"][i] == oracle.STATUS_BAD_TOKEN
    L2 = lengths.copy()
    L2[i] = 99
    assert oracle.verify_left_to_right(target, draft, tokens, L2, T, K, seeds)["status"][i] == oracle.STATUS_BAD_LENGTH
    T2 = T.copy()
    T2[i] = -1.0
    assert (oracle.verify_left_to_right(target, draft, tokens, lengths, T2, K, seeds)["status"][i]
            == oracle.STATUS_BAD_TEMPERATURE)
