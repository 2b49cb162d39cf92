"""The comparison helpers the GPU parity tests rely on, checked on the CPU: the pooled oracle
equals the plain one, and the admissible-outcome rule for flagged draws allows exactly the
outcomes a draw on the other side of its window gives (and nothing else)."""

import numpy as np
import pytest

import oracle
from parity import HostInputs, admissible_outcomes, compare_verify, run_oracle_pooled
from workloads import make_workload


def _h(w, **kw):
    return HostInputs.of_workload(w, **kw)


@pytest.mark.parametrize("name,kw", [("mixed", dict(B=10, gamma=3, V=3001, seed=3)),
                                     ("mid", dict(B=9, gamma=4, V=2048, seed=4)),
                                     ("greedy", dict(B=12, gamma=5, V=999, seed=5))])
def test_pooled_oracle_equals_the_plain_one(name, kw):
    w = make_workload(name, "cpu", **kw)
    h = _h(w)
    a = run_oracle_pooled(h, block=3, workers=2)
    if h.draft is None:
        b = oracle.verify_greedy(w.target, w.draft_tokens)
    else:
        b = oracle.verify(w.target, w.draft, w.draft_tokens, None, w.temperature, w.top_k, w.seed)
    for k in b:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_admissible_outcomes_of_unflagged_requests_are_the_oracles():
    w = make_workload("mixed", "cpu", B=16, gamma=4, V=2000, seed=6)
    h = _h(w)
    ref = oracle.verify(w.target, w.draft, w.draft_tokens, None, w.temperature, w.top_k, w.seed)
    for i in range(w.B):
        if ref["emit_flag"][i] or ref["accept_flags"][i]:
            continue
        n = int(ref["num_accepted"][i])
        assert admissible_outcomes(h, i) == {(n, int(ref["out_tokens"][i, n]))}


def _two_token(t_logits, d_logits, x, L, seed):
    """One request over a two-token vocabulary, fp64 logits (exact in the oracle)."""
    t = np.asarray(t_logits, dtype=np.float64)[None]
    d = np.asarray(d_logits, dtype=np.float64)[None]
    return HostInputs.of(t, d, np.asarray(x)[None], np.asarray([L]), np.ones(1), np.zeros(1), np.asarray([seed],
                                                                                                       dtype=np.uint64))


def test_flagged_acceptance_admits_both_decisions():
    seed = 12345
    u_acc, u_res = oracle.uniforms(np.uint64(seed), np.uint64(0), np.arange(2))
    # p_d(0) = 1/2 and p_t(0) = r/2, so that r = min(1, p_t/p_d) lies 4e-7 above u_acc(0)
    r = float(u_acc[0]) + 4e-7
    a = np.log(r / (2.0 - r))
    h = _two_token([[a, 0.0], [0.0, 0.0]], [[0.0, 0.0]], [0], 1, seed)
    ref = oracle.verify(h.target, h.draft, h.tokens, h.lengths, h.temperature, h.top_k, h.seed)
    assert ref["accept_flags"][0] == 1 and ref["num_accepted"][0] == 1
    adm = admissible_outcomes(h, 0)
    assert {n for n, _ in adm} == {0, 1}
    # a rejection at 0 draws from the residual max(0, p_t - p_d), all of it on token 1
    assert (0, 1) in adm and (0, 0) not in adm
    # compare_verify: the oracle's outcome, the other admissible one, and one that is not
    ok = dict(num_accepted=np.array([1]), out_tokens=np.array([[0, int(ref["out_tokens"][0, 1])]]),
              status=np.array([0]))
    compare_verify(ok, ref, inputs=h, check_prob=False)
    other = dict(num_accepted=np.array([0]), out_tokens=np.array([[1, -1]]), status=np.array([0]))
    assert compare_verify(other, ref, inputs=h, check_prob=False)["admissible"] == 1
    wrong = dict(num_accepted=np.array([0]), out_tokens=np.array([[0, -1]]), status=np.array([0]))
    with pytest.raises(AssertionError):
        compare_verify(wrong, ref, inputs=h, check_prob=False)


def test_flagged_emit_admits_the_neighbouring_token():
    seed = 777
    u_acc, u_res = oracle.uniforms(np.uint64(seed), np.uint64(0), np.arange(1))
    # L = 0: a fresh token from target row 0 with p(0) = u_res(0) + 3e-11, so u * W lies just
    # below the boundary between tokens 0 and 1
    p0 = float(u_res[0]) + 3e-11
    h = _two_token([[np.log(p0), np.log1p(-p0)], [0.0, 0.0]], [[0.0, 0.0]], [0], 0, seed)
    ref = oracle.verify(h.target, h.draft, h.tokens, h.lengths, h.temperature, h.top_k, h.seed)
    assert ref["emit_flag"][0]
    assert admissible_outcomes(h, 0) == {(0, 0), (0, 1)}


def test_unflagged_mismatch_fails():
    w = make_workload("tiny", "cpu", B=8, gamma=4, V=500, seed=9)
    ref = oracle.verify(w.target, w.draft, w.draft_tokens, None, w.temperature, None, w.seed)
    gpu = dict(num_accepted=ref["num_accepted"].copy(), out_tokens=ref["out_tokens"].copy(),
               status=ref["status"].copy(), accept_prob=ref["accept_prob"].astype(np.float32))
    i = int(np.nonzero(~(ref["emit_flag"] | (ref["accept_flags"] > 0)))[0][0])
    n = int(gpu["num_accepted"][i])
    gpu["out_tokens"][i, n] = (gpu["out_tokens"][i, n] + 1) % 500
    with pytest.raises(AssertionError):
        compare_verify(gpu, ref, inputs=_h(w))


def test_flag_bound_is_asserted():
    w = make_workload("tiny", "cpu", B=4, gamma=4, V=500, seed=10)
    ref = oracle.verify(w.target, w.draft, w.draft_tokens, None, w.temperature, None, w.seed)
    gpu = dict(num_accepted=ref["num_accepted"], out_tokens=ref["out_tokens"], status=ref["status"])
    compare_verify(gpu, ref, check_prob=False, bound=True)
    ref2 = dict(ref, accept_flags=ref["accept_flags"] + 1)      # a flag per request: far above 1e-4
    with pytest.raises(AssertionError):
        compare_verify(gpu, ref2, check_prob=False, bound=True)
