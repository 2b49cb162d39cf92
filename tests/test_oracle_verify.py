"""Pins of the verification oracle to facts outside itself.

* losslessness: emitted tokens follow the target distribution (chi-square over
  10^6 trials on tiny vocabularies), position by position and for the bonus row;
* the closed form of the expected number of accepted drafts,
  sum_k prod_{j<=k} sum_x min(p_t,j(x), p_d,j(x));
* identical target and draft distributions accept every draft;
* the worked example of the DSpark paper's appendix counterexample
  (acceptance rate 0.8; residual mass on A);
* log-probabilities against scipy's logsumexp; top-k kept sets against
  constructed ties; the inverse CDF against floor(u * V) for uniform weights;
* greedy verification against constructed argmax mismatches and ties;
* status words for bad data.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import verification as ov

N_TRIALS = 1_000_000
P_MIN = 1e-4


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _fixed_rows_inputs(pt, pd, n, rng):
    """Every trial shares per-position target pt[G+1, V] and draft pd[G, V] distributions;
    draft tokens are drawn from pd by an RNG independent of the verifier's draws."""
    G = pd.shape[0]
    target = np.broadcast_to(np.log(pt), (n,) + pt.shape)
    draft = np.broadcast_to(np.log(pd), (n,) + pd.shape)
    toks = np.stack([rng.choice(pd.shape[1], size=n, p=pd[k]) for k in range(G)], axis=1) \
        if G else np.zeros((n, 0), dtype=np.int64)
    return target, draft, toks


def _chi2_ok(tokens, p):
    obs = np.bincount(tokens, minlength=len(p))
    exp = p * len(tokens)
    return stats.chisquare(obs, exp).pvalue


@pytest.mark.parametrize("V", [2, 3, 8])
def test_lossless_per_position_chi_square(V):
    rng = np.random.default_rng(100 + V)
    G = 2
    pt = _softmax(rng.normal(0, 1.0, (G + 1, V)))
    pd = _softmax(rng.normal(0, 1.0, (G, V)))
    target, draft, toks = _fixed_rows_inputs(pt, pd, N_TRIALS, rng)
    out = oracle.verify(target, draft, toks)
    n = out["num_accepted"]
    ot = out["out_tokens"]
    assert (out["status"] == 0).all()
    for k in range(G + 1):
        reached = n >= k
        pval = _chi2_ok(ot[reached, k], pt[k])
        assert pval > P_MIN, (V, k, pval)


def test_expected_accepted_length_closed_form():
    rng = np.random.default_rng(5)
    V, G = 6, 4
    pt = _softmax(rng.normal(0, 1.0, (G + 1, V)))
    pd = _softmax(rng.normal(0, 1.0, (G, V)))
    alpha = np.minimum(pt[:G], pd).sum(axis=1)
    expected = sum(np.prod(alpha[: k + 1]) for k in range(G))
    target, draft, toks = _fixed_rows_inputs(pt, pd, N_TRIALS, rng)
    n = oracle.verify(target, draft, toks)["num_accepted"].astype(np.float64)
    se = n.std() / math.sqrt(len(n))
    assert abs(n.mean() - expected) < 5 * se, (n.mean(), expected, se)


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(9)
    B, G, V = 64, 5, 300
    z = rng.normal(0, 3, (B, G + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, (B, G))
    out = oracle.verify(z, z[:, :G].copy(), toks, temperature=np.full(B, 0.8))
    assert (out["num_accepted"] == G).all()
    assert (out["accept_prob"] == 1.0).all()
    assert (out["out_tokens"][:, :G] == toks).all()


def test_identical_distributions_bonus_follows_target():
    rng = np.random.default_rng(10)
    V, G = 5, 3
    pt = _softmax(rng.normal(0, 1.0, (G + 1, V)))
    pd = pt[:G].copy()
    target, draft, toks = _fixed_rows_inputs(pt, pd, N_TRIALS // 4, rng)
    out = oracle.verify(target, draft, toks)
    assert (out["num_accepted"] == G).all()
    assert _chi2_ok(out["out_tokens"][:, G], pt[G]) > P_MIN


def test_appendix_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "appendix_counterexample.json")))
    pt = np.array([g["p_target"], [0.5, 0.5]])
    pd = np.array([g["p_draft"]])
    # acceptance rate = sum_x min(p_t, p_d)
    assert abs(np.minimum(pt[0], pd[0]).sum() - g["sum_min"]) < 1e-12
    rng = np.random.default_rng(3)
    target, draft, toks = _fixed_rows_inputs(pt, pd, 400_000, rng)
    out = oracle.verify(target, draft, toks)
    r = out["accept_prob"][:, 0]
    assert np.allclose(r[toks[:, 0] == 0], g["accept_prob_A"], rtol=0, atol=1e-15)
    assert np.allclose(r[toks[:, 0] == 1], 0.3 / 0.5, rtol=0, atol=1e-15)
    acc = (out["num_accepted"] == 1).mean()
    assert abs(acc - g["sum_min"]) < 5 * math.sqrt(0.8 * 0.2 / len(r))
    rej = out["num_accepted"] == 0
    # a rejection can only happen on B, and the residual max(0, p_t - p_d) puts all mass on A
    assert (toks[rej, 0] == 1).all() and (out["out_tokens"][rej, 0] == 0).all()
    first = out["out_tokens"][:, 0]
    assert _chi2_ok(first, np.array(g["lossless_output"])) > P_MIN


def test_zero_length_emits_a_fresh_target_token():
    rng = np.random.default_rng(12)
    V, G = 4, 3
    pt = _softmax(rng.normal(0, 1.0, (G + 1, V)))
    pd = _softmax(rng.normal(0, 1.0, (G, V)))
    n = 300_000
    target, draft, toks = _fixed_rows_inputs(pt, pd, n, rng)
    out = oracle.verify(target, draft, toks, lengths=np.zeros(n, dtype=np.int64))
    assert (out["num_accepted"] == 0).all()
    assert np.isnan(out["accept_prob"]).all()
    assert (out["out_tokens"][:, 1:] == -1).all()
    assert _chi2_ok(out["out_tokens"][:, 0], pt[0]) > P_MIN


def test_variable_lengths_bonus_row_is_row_L():
    rng = np.random.default_rng(13)
    V, G = 4, 3
    pt = _softmax(rng.normal(0, 2.0, (G + 1, V)))
    pd = pt[:G].copy()          # everything accepted, so row L decides the last token
    n = 200_000
    target, draft, toks = _fixed_rows_inputs(pt, pd, n, rng)
    L = rng.integers(0, G + 1, n)
    out = oracle.verify(target, draft, toks, lengths=L)
    assert (out["num_accepted"] == L).all()
    for l in range(G + 1):
        sel = L == l
        assert _chi2_ok(out["out_tokens"][sel, l], pt[l]) > P_MIN


def test_log_probs_against_scipy_logsumexp():
    rng = np.random.default_rng(14)
    for T in (0.6, 1.0, 1.3):
        z = rng.normal(0, 3, (8, 1000)).astype(np.float32)
        lp = oracle.log_probs(z, T)
        ref = z.astype(np.float64) / T - special.logsumexp(z.astype(np.float64) / T, axis=1, keepdims=True)
        assert np.allclose(lp, ref, rtol=0, atol=1e-12)
        assert np.allclose(np.exp(lp).sum(axis=1), 1.0, atol=1e-12)


def test_top_k_kept_set_keeps_ties():
    z = np.array([[5.0, 4.0, 1.0, 4.0, 4.0, -2.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
                  [3.0, 2.0, 1.0, 0.0, -1.0, -2.0]])
    keep = oracle.kept_mask(z, np.array([3, 2, 3]))
    assert keep[0].tolist() == [True, True, False, True, True, False]   # 4 kept: tie at the cut
    assert keep[1].all()
    assert keep[2].tolist() == [True, True, True, False, False, False]
    assert oracle.kept_mask(z, 0).all() and oracle.kept_mask(z, 6).all() and oracle.kept_mask(z, 99).all()
    lp = oracle.log_probs(z[2], 0.5, 3)
    ref = z[2, :3] / 0.5 - special.logsumexp(z[2, :3] / 0.5)
    assert np.allclose(lp[:3], ref, atol=1e-13) and np.isneginf(lp[3:]).all()


def test_top_k_temperature_output_follows_tempered_target():
    rng = np.random.default_rng(15)
    V, G, K, T = 8, 1, 3, 0.7
    zt = rng.normal(0, 1.0, (G + 1, V))
    zd = zt[:G] + rng.normal(0, 0.8, (G, V))
    n = 500_000
    pd = np.exp(oracle.log_probs(zd, T, K))
    target = np.broadcast_to(zt, (n, G + 1, V))
    draft = np.broadcast_to(zd, (n, G, V))
    toks = rng.choice(V, size=(n, 1), p=pd[0])
    out = oracle.verify(target, draft, toks, temperature=np.full(n, T), top_k=np.full(n, K))
    pt0 = np.exp(oracle.log_probs(zt[0], T, K))
    first = out["out_tokens"][:, 0]
    assert set(np.unique(first)) <= set(np.nonzero(pt0 > 0)[0])
    keep = pt0 > 0
    obs = np.bincount(first, minlength=V)[keep]
    assert stats.chisquare(obs, pt0[keep] * n).pvalue > P_MIN


def test_inverse_cdf_uniform_weights_is_floor():
    V = 16
    w = np.full(V, 1.0 / V)
    ww = np.broadcast_to(w, (V, V))
    tok, W, flagged = ov.inverse_cdf(ww, np.arange(V) / V)          # exactly on each boundary
    assert tok.tolist() == list(range(V)) and flagged.all() and np.allclose(W, 1.0)
    tok, _, flagged = ov.inverse_cdf(ww, (np.arange(V) + 0.5) / V)
    assert tok.tolist() == list(range(V)) and not flagged.any()
    tok, _, _ = ov.inverse_cdf(np.array([[0.0, 0.3, 0.0, 0.7, 0.0]]), np.array([1.0 - 2 ** -53]))
    assert tok[0] == 3


def _complement_inputs(B, G, V, S_size, seed):
    """Target rows uniform (all logits 0); draft rows uniform on a random set S of S_size tokens
    (logit 0 there, -inf elsewhere); draft tokens drawn from S."""
    rng = np.random.default_rng(seed)
    target = np.zeros((B, G + 1, V), dtype=np.float32)
    draft = np.full((B, G, V), -np.inf, dtype=np.float32)
    sets = np.empty((B, G, S_size), dtype=np.int64)
    tokens = np.empty((B, G), dtype=np.int64)
    for i in range(B):
        for k in range(G):
            S = np.sort(rng.choice(V, size=S_size, replace=False))
            sets[i, k] = S
            draft[i, k, S] = 0.0
            tokens[i, k] = S[rng.integers(S_size)]
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    return target, draft, tokens, sets, seeds


def complement_token(V, S, u):
    """The closed form of the emitted token when p_t is uniform over V tokens and p_d uniform over
    S: the residual max(0, 1/V - 1/|S|) is 1/V on the complement of S and 0 on S, so the inverse CDF
    in ascending order at u lands on the complement token of rank floor(u * (V - |S|))."""
    comp = np.setdiff1d(np.arange(V), S)
    return int(comp[int(np.floor(u * len(comp)))])


def test_residual_closed_form_at_large_vocabulary():
    """At V = 151936: uniform target against a draft uniform on |S| = 1519 tokens.  Every acceptance
    ratio is |S| / V; after a rejection the token is the complement token of rank
    floor(u * (V - |S|)); after full acceptance it is floor(u * V).  Pins the residual, its
    normalisation and the inverse CDF at the vocabulary size of the workloads."""
    B, G, V, Ss = 8, 3, 151936, 1519
    target, draft, tokens, sets, seeds = _complement_inputs(B, G, V, Ss, 41)
    out = oracle.verify(target, draft, tokens, seed=seeds)
    assert (out["status"] == 0).all()
    r = Ss / V
    seen_rej = seen_all = 0
    for i in range(B):
        n = int(out["num_accepted"][i])
        np.testing.assert_allclose(out["accept_prob"][i, :], r, rtol=1e-12)
        u_acc, u_emit = oracle.uniforms(np.full(G + 1, seeds[i], dtype=np.int64).view(np.uint64),
                                        np.full(G + 1, i), np.arange(G + 1))
        # the acceptance tests themselves: u < |S| / V
        first_rej = next((k for k in range(G) if not u_acc[k] < r), G)
        assert n == first_rej
        want = complement_token(V, sets[i, n], u_emit[n]) if n < G else int(np.floor(u_emit[G] * V))
        assert int(out["out_tokens"][i, n]) == want or out["emit_flag"][i]
        seen_rej += n < G
        seen_all += n == G
    assert seen_rej > 0


def test_greedy_constructed_mismatch_and_ties():
    rng = np.random.default_rng(16)
    B, G, V = 40, 6, 50
    z = rng.normal(0, 1, (B, G + 1, V)).astype(np.float32)
    peak = rng.integers(0, V, (B, G + 1))
    z[np.arange(B)[:, None], np.arange(G + 1)[None, :], peak] = 10.0      # unique planted max
    m = rng.integers(0, G + 1, B)                                        # first mismatch (G = none)
    toks = peak[:, :G].copy()
    for i in range(B):
        if m[i] < G:
            toks[i, m[i]] = (peak[i, m[i]] + 1) % V
            toks[i, m[i] + 1:] = rng.integers(0, V, G - m[i] - 1)
    out = oracle.verify_greedy(z, toks)
    assert (out["num_accepted"] == m).all()
    for i in range(B):
        assert out["out_tokens"][i, : m[i]].tolist() == peak[i, : m[i]].tolist()
        assert out["out_tokens"][i, m[i]] == peak[i, m[i]]
    # tie: two equal maxima, the lower id is the argmax; the higher id is a mismatch
    zt = np.zeros((1, 2, 8), dtype=np.float32)
    zt[0, 0, [2, 5]] = 3.0
    zt[0, 1, 1] = 1.0
    out = oracle.verify_greedy(zt, np.array([[5]]))
    assert out["num_accepted"][0] == 0 and out["out_tokens"][0].tolist() == [2, -1]
    out = oracle.verify_greedy(zt, np.array([[2]]))
    assert out["num_accepted"][0] == 1 and out["out_tokens"][0].tolist() == [2, 1]


def test_greedy_generator_expected_length():
    import torch  # noqa: F401
    from workloads import make_workload
    w = make_workload("greedy", "cpu", B=20000, gamma=6, V=64, seed=77)
    out = oracle.verify_greedy(w.target, w.draft_tokens)
    n = out["num_accepted"].astype(np.float64)
    V, G = 64, 6
    q = np.array([0.9 ** j + (1 - 0.9 ** j) / V for j in range(1, G + 1)])
    expected = sum(np.prod(q[: k + 1]) for k in range(G))
    se = n.std() / math.sqrt(len(n))
    assert abs(n.mean() - expected) < 5 * se, (n.mean(), expected)


def test_status_words():
    rng = np.random.default_rng(17)
    B, G, V = 8, 3, 20
    t = rng.normal(0, 1, (B, G + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, (B, G, V)).astype(np.float32)
    toks = rng.integers(0, V, (B, G))
    T = np.ones(B)
    L = np.full(B, G)
    toks[0, 1] = V                      # out of range
    T[1] = -1.0                         # negative temperature
    t[2, 0, 3] = np.nan                 # NaN in a needed target row
    L[3] = 1
    t[3, 3, 0] = np.nan                 # NaN beyond the verify length: not needed, fine
    L[4] = G + 1                        # bad length
    d[5, 2, 0] = np.inf                 # +inf in a needed draft row
    T[6] = np.nan
    t[7, 2, :] = -np.inf                # a needed row with no finite logit (reading R22)
    out = oracle.verify(t, d, toks, lengths=L, temperature=T)
    st = out["status"]
    assert st[0] == ov.STATUS_BAD_TOKEN
    assert st[1] == ov.STATUS_BAD_TEMPERATURE
    assert st[2] == ov.STATUS_NONFINITE
    assert st[3] == 0
    assert st[7] == ov.STATUS_NONFINITE
    assert st[4] == ov.STATUS_BAD_LENGTH
    assert st[5] == ov.STATUS_NONFINITE
    assert st[6] & ov.STATUS_BAD_TEMPERATURE
    bad = st != 0
    assert (out["num_accepted"][bad] == 0).all() and (out["out_tokens"][bad] == -1).all()
