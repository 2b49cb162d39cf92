"""Pins of the scheduler oracle.

* the numbers printed in the DSpark paper's appendix counterexample
  (Theta_0 = 1.0, Theta_1 = 0.9, Theta_2 = 1.134 / 0.81; global search picks
  2 / 0; early stop picks 0);
* global mode equals brute-force enumeration of all length vectors (B <= 4);
* early stop never beats brute force and matches it when Theta is unimodal
  along the sorted path;
* for a fixed batch size the sorted top-m pool maximises expected accepted
  tokens (the exchange argument of §3.2.2), by brute force;
* end to end, the retrospective (global) scheduler driven by a confidence
  that depends on the first draft token yields (0.85, 0.15) while the
  early-stop scheduler keeps the lossless (0.7, 0.3).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.scheduling import MODE_EARLY_STOP, MODE_GLOBAL, ONE, fixed_point, survival


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "appendix_counterexample.json")))


def _sps_from(g, n=8):
    sps = np.zeros(n)
    for b, v in g["sps"].items():
        sps[int(b)] = v
    return sps


@pytest.mark.parametrize("case", ["case_high", "case_low"])
def test_appendix_theta_values(golden_dir, case):
    g = _golden(golden_dir)
    sps = _sps_from(g)
    conf = np.array([[g["a1"], g[case]["c2"]]], dtype=np.float32)
    path, pool, a = oracle.theta_path(conf, sps, budget=3)
    tol = 1e-6          # the confidences are float32 values of the printed decimals
    assert abs(path[0] - g["theta0"]) < tol
    assert abs(path[1] - g["theta1"]) < tol
    if g[case]["a2"] > 0:
        assert abs(a[0, 1] - g[case]["a2"]) < tol
        assert abs(path[2] - g[case]["theta2"]) < tol
    else:
        # a = 0 is never a candidate; Theta at length 2 is still (1 + 0.8 + 0) * SPS(3)
        assert len(path) == 2
        assert abs((1 + float(a[0, 0])) * sps[3] - g[case]["theta2"]) < tol
    L, _ = oracle.schedule(conf, sps, 3, MODE_GLOBAL)
    assert L[0] == g[case]["global_length"]
    L, th = oracle.schedule(conf, sps, 3, MODE_EARLY_STOP)
    assert L[0] == g["early_stop_length"] and th == path[0]


def _random_problem(rng, R, G):
    conf = rng.uniform(0.3, 1.0, (R, G)).astype(np.float32)
    conf[rng.random((R, G)) < 0.1] = 0.0
    conf[rng.random((R, G)) < 0.05] = 1.0
    n = R * (G + 1) + 1
    b = np.arange(n, dtype=np.float64)
    kind = rng.integers(0, 3)
    if kind == 0:       # smooth concave throughput -> steps/s
        X0 = rng.uniform(2, 20)
        tput = 10.0 * (1 - np.exp(-b / X0))
    elif kind == 1:     # jagged, step-wise
        tput = np.cumsum(rng.uniform(0, 1, n) * (rng.random(n) < 0.5))
    else:
        tput = rng.uniform(0.5, 2.0, n) * b ** rng.uniform(0.2, 0.9)
    sps = np.zeros(n)
    sps[1:] = tput[1:] / b[1:]
    budget = int(rng.integers(R, R * (G + 1) + 2))
    return conf, sps, budget


def test_global_mode_equals_brute_force():
    rng = np.random.default_rng(21)
    for trial in range(300):
        R = int(rng.integers(1, 5))
        G = int(rng.integers(1, 5 if R <= 3 else 4))
        conf, sps, budget = _random_problem(rng, R, G)
        L, th = oracle.schedule(conf, sps, budget, MODE_GLOBAL)
        best, args = oracle.schedule_bruteforce(conf, sps, budget)
        assert th == best, (trial, th, best)
        assert tuple(int(x) for x in L) in args
        assert (L + 1).sum() <= max(budget, R)


def test_early_stop_bounded_by_brute_force_and_exact_when_unimodal():
    rng = np.random.default_rng(22)
    unimodal_seen = 0
    for trial in range(300):
        R = int(rng.integers(1, 5))
        G = int(rng.integers(1, 4))
        conf, sps, budget = _random_problem(rng, R, G)
        L, th = oracle.schedule(conf, sps, budget, MODE_EARLY_STOP)
        best, _ = oracle.schedule_bruteforce(conf, sps, budget)
        assert th <= best
        path, _, _ = oracle.theta_path(conf, sps, budget)
        m = int(L.sum())
        # rises strictly up to m, then the next step does not rise
        assert all(path[i + 1] > path[i] for i in range(m))
        assert m + 1 >= len(path) or path[m + 1] <= path[m]
        peak = int(np.argmax(path))
        unimodal = all(path[i + 1] > path[i] for i in range(peak)) and \
            all(path[i + 1] <= path[i] for i in range(peak, len(path) - 1))
        if unimodal:
            unimodal_seen += 1
            assert th == best
    assert unimodal_seen > 30


def test_stop_on_equal_theta():
    # c = 1 gives a = 1: Theta_1 = 2 * 0.5 = 1.0 = Theta_0, not an improvement
    conf = np.array([[1.0, 1.0]], dtype=np.float32)
    sps = np.array([0.0, 1.0, 0.5, 0.4])
    L, th = oracle.schedule(conf, sps, 3, MODE_EARLY_STOP)
    assert L[0] == 0 and th == 1.0
    L, th = oracle.schedule(conf, sps, 3, MODE_GLOBAL)        # Theta_2 = 3 * 0.4 = 1.2
    assert L[0] == 2 and abs(th - 1.2) < 1e-15


def test_fixed_batch_top_m_pool_is_optimal():
    rng = np.random.default_rng(23)
    for _ in range(100):
        R, G = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        conf = rng.uniform(0.0, 1.0, (R, G)).astype(np.float32)
        a = survival(conf)
        q = [[fixed_point(a[r, j]) for j in range(G)] for r in range(R)]
        pool = oracle.scheduling.candidates(a)
        for m in range(len(pool) + 1):
            top = sum(fixed_point(a[r, j]) for r, j in pool[:m])
            best = -1
            for lens in itertools.product(range(G + 1), repeat=R):
                if sum(lens) != m or any(a[r, l - 1] <= 0 for r, l in enumerate(lens) if l > 0):
                    continue
                best = max(best, sum(sum(q[r][:l]) for r, l in enumerate(lens)))
            assert top == best


def test_survival_is_left_to_right_float32_product():
    rng = np.random.default_rng(24)
    c = rng.uniform(0, 1, (50, 16)).astype(np.float32)
    a = survival(c)
    assert a.dtype == np.float32
    for r in range(50):
        acc = np.float32(1.0)
        for j in range(16):
            acc = np.float32(acc * c[r, j])
            assert a[r, j] == acc
    assert (np.diff(a, axis=1) <= 0).all()          # non-increasing along the block


def test_budget_caps_batch_tokens():
    rng = np.random.default_rng(25)
    R, G = 16, 8
    conf = np.full((R, G), 0.99, dtype=np.float32)
    b = np.arange(R * (G + 1) + 1, dtype=np.float64)
    sps = np.zeros_like(b)
    sps[1:] = 1.0            # throughput grows with every token: admit as many as allowed
    for budget in (R - 3, R, R + 5, R * 3, R * (G + 1), R * (G + 1) + 10):
        L, _ = oracle.schedule(conf, sps, budget, MODE_EARLY_STOP)
        assert (L + 1).sum() <= max(budget, R)
        assert (L + 1).sum() == max(R, min(budget, R * (G + 1)))


def test_retrospective_scheduler_biases_output(golden_dir):
    """End-to-end appendix counterexample, run through both oracles."""
    g = _golden(golden_dir)
    sps = _sps_from(g)
    n = 400_000
    rng = np.random.default_rng(26)
    pt = np.array([g["p_target"], [0.5, 0.5], [0.5, 0.5]])
    pd = np.array([g["p_draft"], [0.5, 0.5]])
    target = np.broadcast_to(np.log(pt), (n, 3, 2))
    draft = np.broadcast_to(np.log(pd), (n, 2, 2))
    toks = np.stack([rng.choice(2, size=n, p=pd[k]) for k in range(2)], axis=1)
    # the confidence of position 2 depends on the realised first draft token
    conf_A = np.array([[g["a1"], g["case_high"]["c2"]]], dtype=np.float32)
    conf_B = np.array([[g["a1"], g["case_low"]["c2"]]], dtype=np.float32)
    for mode, expect in ((MODE_GLOBAL, g["retrospective_output"]), (MODE_EARLY_STOP, g["lossless_output"])):
        lA, _ = oracle.schedule(conf_A, sps, 3, mode)
        lB, _ = oracle.schedule(conf_B, sps, 3, mode)
        L = np.where(toks[:, 0] == 0, lA[0], lB[0])
        out = oracle.verify(target, draft, toks, lengths=L)
        first = out["out_tokens"][:, 0]
        obs = np.bincount(first, minlength=2)
        p = stats.chisquare(obs, np.array(expect) * n).pvalue
        assert p > 1e-4, (mode, obs / n, expect)


def test_fixed_point_is_exact_and_fits_int64():
    """q(a) = floor(a * 2^FRAC_BITS) is a * 2^FRAC_BITS itself for every float32 a >= 2^-24, and the
    largest tau (every request admitted in full at the candidate limit) fits a signed int64."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.random(2000).astype(np.float32),
                        np.float32(2.0) ** -rng.integers(0, 25, 200).astype(np.float32),
                        np.array([1.0, np.nextafter(np.float32(1), np.float32(0))], dtype=np.float32)])
    for x in a:
        if x >= 2.0 ** -24:
            assert Fraction(fixed_point(x)) == Fraction(float(x)) * ONE
    tiny = np.float32(2.0 ** -30) * np.float32(1.5)
    assert fixed_point(tiny) == int(Fraction(float(tiny)) * ONE)   # floor below 2^-24
    max_candidates, max_requests = 16384, 16384
    assert (max_requests + max_candidates) * ONE < 2 ** 63


def test_topk_at_the_global_capacity_is_the_global_schedule():
    """With the current confidences equal to the earlier ones, the asynchronous scheduler admits
    exactly what the global search admits (§5.2 keeps the sort and only moves the capacity)."""
    rng = np.random.default_rng(71)
    for trial in range(30):
        B, G = int(rng.integers(1, 40)), int(rng.integers(1, 9))
        conf = rng.uniform(0.0, 1.0, (B, G)).astype(np.float32)
        conf[rng.random((B, G)) < 0.1] = np.float32(0.75)
        b = np.arange(B * (G + 1) + 1, dtype=np.float64)
        sps = np.zeros_like(b)
        sps[1:] = rng.uniform(0.5, 2.0) * (1 - np.exp(-b[1:] / rng.uniform(1, 10 * B))) / b[1:]
        budget = int(rng.integers(B, B * (G + 1) + 1))
        K = oracle.capacity(conf, sps, budget)
        lg, _ = oracle.schedule(conf, sps, budget, MODE_GLOBAL)
        assert int(lg.sum()) == K
        assert (oracle.schedule_topk(conf, K) == lg).all()


def test_topk_admits_the_most_likely_prefixes():
    """Brute force over prefix-closed admissions of size K: none has a larger total survival than
    the top-K selection (the rank-preserving property of §5.2; fixed-batch optimality of §3.2.2)."""
    rng = np.random.default_rng(72)
    for trial in range(40):
        B, G = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        conf = rng.uniform(0.05, 1.0, (B, G)).astype(np.float32)
        a = survival(conf).astype(np.float64)
        K = int(rng.integers(0, B * G + 2))
        L = oracle.schedule_topk(conf, K)
        assert int(L.sum()) == min(K, B * G)
        got = sum(a[r, :L[r]].sum() for r in range(B))
        best = -1.0
        for lens in itertools.product(range(G + 1), repeat=B):
            if sum(lens) == min(K, B * G):
                best = max(best, sum(a[r, :lens[r]].sum() for r in range(B)))
        assert got >= best - 1e-12


def test_asynchronous_scheduler_keeps_the_target_distribution(golden_dir):
    """The appendix example once more: with the capacity taken from confidences that precede the
    first draft token (two steps earlier) and top-K admission of the current candidates, the first
    output token follows the target (0.7, 0.3) although c_2 depends on x_1 (§5.2)."""
    g = _golden(golden_dir)
    sps = _sps_from(g)
    n = 400_000
    rng = np.random.default_rng(73)
    pt = np.array([g["p_target"], [0.5, 0.5], [0.5, 0.5]])
    pd = np.array([g["p_draft"], [0.5, 0.5]])
    target = np.broadcast_to(np.log(pt), (n, 3, 2))
    draft = np.broadcast_to(np.log(pd), (n, 2, 2))
    toks = np.stack([rng.choice(2, size=n, p=pd[k]) for k in range(2)], axis=1)
    conf_A = np.array([[g["a1"], g["case_high"]["c2"]]], dtype=np.float32)
    conf_B = np.array([[g["a1"], g["case_low"]["c2"]]], dtype=np.float32)
    # the earlier step saw either realisation with the draft's probabilities; its capacity
    # cannot know which one the current step drew
    hist = np.where(rng.random(n) < 0.5, 0, 1)
    K = np.array([oracle.capacity(conf_A, sps, 3), oracle.capacity(conf_B, sps, 3)])[hist]
    LA = [int(oracle.schedule_topk(conf_A, k)[0]) for k in (0, 1, 2)]
    LB = [int(oracle.schedule_topk(conf_B, k)[0]) for k in (0, 1, 2)]
    L = np.where(toks[:, 0] == 0, np.take(LA, K), np.take(LB, K))
    out = oracle.verify(target, draft, toks, lengths=L)
    obs = np.bincount(out["out_tokens"][:, 0], minlength=2)
    assert stats.chisquare(obs, np.array(g["lossless_output"]) * n).pvalue > 1e-4, obs / n
