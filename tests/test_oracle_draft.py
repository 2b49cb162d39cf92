"""Pins of the draft-sampler oracle: the Markov head (DSpark paper, §3.1, Eq. 4 and Eq. 5) and the
confidence head (§3.2.1, Eq. 7)."""

import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle.drafting import markov_draft, round_bf16
from oracle.philox import draft_uniform

NEG = -np.inf


def test_round_bf16_matches_torch_conversion():
    """Round-to-nearest-even to 8 significant bits equals torch's float32 -> bfloat16 conversion
    (a library routine) on random values, exact midpoints and their neighbours."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    mids = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    allb = np.concatenate([bits, mids, mids + np.uint32(1), mids - np.uint32(1)])
    x = allb.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) > 2.0 ** -120) & (np.abs(x) < 3.0e38)]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to 1
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_transition_orientation():
    """W1 = I and W2 = M make the bias of Eq. 5 row x_{k-1} of M; with U = 0 and T = 0 the draft
    follows the argmax of that row.  M[a, s(a)] = 1: the chain follows the map s (a transposed
    operand would follow its inverse)."""
    s = [3, 0, 5, 1, 2, 4]
    V = r = 6
    M = np.zeros((V, V))
    M[np.arange(V), s] = 1.0
    W1, W2t = np.eye(V), M.T.copy()
    G = 7
    out = markov_draft(np.zeros((1, G, V)), W1, W2t, [2], temperature=[0.0])
    want, x = [], 2
    for _ in range(G):
        x = s[x]
        want.append(x)
    assert out["tokens"][0].tolist() == want
    assert (out["status"] == 0).all()
    # the logits are U_k + M[x_{k-1}]
    assert np.array_equal(out["logits"][0, 0], M[2])


def test_of_course_no_problem_joint():
    """§3.1's example: position 1 chooses "of" or "no" evenly, position 2 "course" or "problem"
    evenly; the Markov head adds +-beta for the coherent / incoherent pairs.  Eq. 4 then gives
    P(of, course) = P(no, problem) = sigmoid(2 beta) / 2; empirical frequencies over many requests
    (independent draws) agree within 5 sigma."""
    OF, NO, COURSE, PROBLEM, ANCHOR = 0, 1, 2, 3, 4
    V, beta, B = 5, 1.0, 6000
    W1 = np.zeros((V, 2))
    W1[OF], W1[NO] = [1, 0], [0, 1]
    W2t = np.zeros((V, 2))
    W2t[COURSE], W2t[PROBLEM] = [beta, -beta], [-beta, beta]
    U = np.full((B, 2, V), NEG)
    U[:, 0, [OF, NO]] = 0.0
    U[:, 1, [COURSE, PROBLEM]] = 0.0
    out = markov_draft(U, W1, W2t, np.full(B, ANCHOR), seed=np.full(B, 99, dtype=np.uint64))
    t = out["tokens"]
    p = expit(2 * beta) / 2
    for pair, prob in [((OF, COURSE), p), ((NO, PROBLEM), p), ((OF, PROBLEM), 0.5 - p),
                       ((NO, COURSE), 0.5 - p)]:
        f = np.mean((t[:, 0] == pair[0]) & (t[:, 1] == pair[1]))
        assert abs(f - prob) < 5 * math.sqrt(prob * (1 - prob) / B), (pair, f, prob)


def test_sampling_frequencies_follow_softmax():
    """x_1 over many independent requests with the same logits follows softmax(z / T): a
    chi-square statistic below the 0.9999 quantile for 7 degrees of freedom (~29.9)."""
    rng = np.random.default_rng(8)
    V, B, T = 8, 20000, 0.7
    z = round_bf16(rng.normal(0, 1, V))
    U = np.broadcast_to(z, (B, 1, V))
    out = markov_draft(U, np.zeros((V, 16)), np.zeros((V, 16)), np.zeros(B, dtype=int),
                       temperature=np.full(B, T), seed=np.arange(B, dtype=np.uint64) * 7919)
    p = np.exp(z / T - np.max(z / T))
    p /= p.sum()
    cnt = np.bincount(out["tokens"][:, 0], minlength=V)
    chi2 = ((cnt - B * p) ** 2 / (B * p)).sum()
    assert chi2 < 29.9, chi2


def test_inverse_cdf_order_and_zero_weights():
    """Logits (0, -inf, 0, 0): p = (1/3, 0, 1/3, 1/3).  The draw picks 0 for u < 1/3, 2 for
    u < 2/3, else 3 (ascending token order, zero-weight tokens skipped)."""
    B = 400
    U = np.tile(np.array([0.0, NEG, 0.0, 0.0]), (B, 1, 1))
    seeds = np.arange(B, dtype=np.uint64) + 5
    out = markov_draft(U, np.zeros((4, 16)), np.zeros((4, 16)), np.zeros(B, dtype=int), seed=seeds)
    u = draft_uniform(seeds, np.arange(B), 0)
    want = np.where(u < 1 / 3, 0, np.where(u < 2 / 3, 2, 3))
    assert np.array_equal(out["tokens"][:, 0], want)


def test_low_temperature_is_argmax_and_greedy_ties():
    rng = np.random.default_rng(4)
    B, V = 50, 40
    U = round_bf16(rng.normal(0, 1, (B, 3, V)))
    U[:, :, 7] = 20.0
    out = markov_draft(U, np.zeros((V, 16)), np.zeros((V, 16)), np.zeros(B, dtype=int),
                       temperature=np.full(B, 1e-3), seed=np.arange(B, dtype=np.uint64))
    assert (out["tokens"] == 7).all()
    # greedy: the first of equal maxima
    U2 = np.zeros((1, 2, 5))
    U2[0, :, 1] = U2[0, :, 3] = 2.0
    out = markov_draft(U2, np.zeros((5, 16)), np.zeros((5, 16)), [0], temperature=[0.0])
    assert out["tokens"][0].tolist() == [1, 1]


def test_confidence_head_without_hidden_states():
    """d = 0: Eq. 7 reduces to sigmoid(w . W1[x_{k-1}])."""
    V, r = 12, 16
    W1 = round_bf16(np.random.default_rng(2).normal(0, 1, (V, r)))
    w = np.zeros(r)
    w[3] = 1.0
    out = markov_draft(np.zeros((2, 3, V)), W1, np.zeros((V, r)), [4, 7], temperature=[0.0, 0.0], conf_w=w)
    prev = np.concatenate([[[4], [7]], out["tokens"][:, :-1]], axis=1)
    assert np.allclose(out["conf"], expit(W1[prev, 3]), rtol=1e-15, atol=0)


def test_confidence_temperatures():
    """Per-position temperatures divide the head's logit: conf(tau) = sigmoid(logit(conf(1)) / tau)."""
    rng = np.random.default_rng(12)
    B, G, V, r, d = 4, 3, 50, 16, 8
    U = round_bf16(rng.normal(0, 2, (B, G, V)))
    W1 = round_bf16(rng.normal(0, 1, (V, r)))
    W2t = round_bf16(rng.normal(0, 0.1, (V, r)))
    h = rng.normal(0, 1, (B, G, d))
    w = rng.normal(0, 0.5, d + r)
    kw = dict(seed=np.arange(B, dtype=np.uint64), hidden=h, conf_w=w)
    plain = markov_draft(U, W1, W2t, np.arange(B), **kw)
    tau = np.array([2.0, 0.5, 1.3])
    cal = markov_draft(U, W1, W2t, np.arange(B), conf_tau=tau, **kw)
    assert np.array_equal(plain["tokens"], cal["tokens"])
    t = np.log(plain["conf"] / (1 - plain["conf"]))
    assert np.allclose(cal["conf"], expit(t / tau), rtol=1e-12, atol=0)


def test_confidence_head_picks_concatenation_parts():
    """Eq. 7 with w a basis vector: c_k = sigmoid(h_k[j]) for j < d, and
    sigmoid(W1[x_{k-1}, j - d]) beyond (x_0 = the anchor), against scipy's expit."""
    rng = np.random.default_rng(5)
    B, G, V, r, d = 3, 4, 30, 16, 5
    U = round_bf16(rng.normal(0, 2, (B, G, V)))
    W1 = round_bf16(rng.normal(0, 1, (V, r)))
    W2t = round_bf16(rng.normal(0, 0.1, (V, r)))
    h = rng.normal(0, 1, (B, G, d))
    anchor = rng.integers(0, V, B)
    for j in [0, 3, d, d + 7]:
        w = np.zeros(d + r)
        w[j] = 1.0
        out = markov_draft(U, W1, W2t, anchor, seed=np.arange(B, dtype=np.uint64), hidden=h, conf_w=w)
        prev = np.concatenate([anchor[:, None], out["tokens"][:, :-1]], axis=1)
        want = expit(h[:, :, j]) if j < d else expit(W1[prev, j - d])
        assert np.allclose(out["conf"], want, rtol=1e-15, atol=0)


def test_status_words():
    B, G, V = 5, 3, 20
    U = np.zeros((B, G, V))
    U[2, 1, 4] = np.nan          # bad row at step 1
    U[3, 0, :] = NEG             # no finite logit at step 0
    out = markov_draft(U, np.zeros((V, 16)), np.zeros((V, 16)), [0, -1, 0, 0, V],
                       temperature=[np.nan, 1.0, 1.0, 1.0, 1.0])
    assert out["status"].tolist() == [oracle.STATUS_BAD_TEMPERATURE, oracle.STATUS_BAD_TOKEN,
                                      oracle.STATUS_NONFINITE, oracle.STATUS_NONFINITE,
                                      oracle.STATUS_BAD_TOKEN]
    assert (out["tokens"] == -1).all() and np.isnan(out["conf"]).all()


def test_drafts_verified_against_themselves_are_all_accepted():
    """Lossless pairing: when the target distribution equals the draft one (the target rows are
    the stored draft logits), every acceptance ratio is 1 and the whole block is accepted."""
    rng = np.random.default_rng(6)
    B, G, V, r = 4, 5, 300, 32
    U = round_bf16(rng.normal(0, 2, (B, G, V)))
    W1 = round_bf16(rng.normal(0, 1, (V, r)))
    W2t = round_bf16(rng.normal(0, 0.2, (V, r)))
    T = np.array([1.0, 0.5, 0.0, 1.3])
    out = markov_draft(U, W1, W2t, rng.integers(0, V, B), temperature=T, seed=np.arange(B, dtype=np.uint64))
    target = np.concatenate([out["logits"], round_bf16(rng.normal(0, 2, (B, 1, V)))], axis=1)
    v = oracle.verify(target, out["logits"], out["tokens"], temperature=T, seed=np.arange(B, dtype=np.uint64) + 100)
    assert (v["num_accepted"] == G).all()
    assert (v["accept_prob"] == 1.0).all()
