"""Pins of the overlap-mass oracle, c*_k = sum_v min(p_t, p_d) (DSpark paper, §3.2.1, Eq. 8)."""

import json
import math
import os

import numpy as np

import oracle
from oracle.overlap import overlap_mass


def _softmax(z, T=1.0):
    y = np.asarray(z, dtype=np.float64) / T
    e = np.exp(y - y.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_total_variation_identity():
    """Eq. 8 also writes the overlap as 1 - (1/2) ||p_t - p_d||_1: check the oracle against that
    form, with temperatures, on rows computed here with a plain softmax."""
    rng = np.random.default_rng(51)
    B, G, V = 6, 4, 300
    t = rng.normal(0, 3, (B, G + 1, V)).astype(np.float32)
    d = (t[:, :G] + rng.normal(0, 1.5, (B, G, V))).astype(np.float32)
    T = rng.uniform(0.5, 2.0, B)
    c = overlap_mass(t, d, temperature=T)["overlap"]
    for i in range(B):
        pt = _softmax(t[i, :G], T[i])
        pd = _softmax(d[i], T[i])
        tv = 1.0 - 0.5 * np.abs(pt - pd).sum(axis=-1)
        assert np.allclose(c[i], tv, rtol=0, atol=1e-13)


def test_appendix_overlap(golden_dir):
    """The appendix pair (0.7, 0.3) against (0.5, 0.5): overlap 0.8 as printed."""
    g = json.load(open(os.path.join(golden_dir, "appendix_counterexample.json")))
    t = np.log(np.array([[g["p_target"], [0.5, 0.5]]]))
    d = np.log(np.array([[g["p_draft"]]]))
    c = overlap_mass(t, d)["overlap"]
    assert abs(c[0, 0] - g["sum_min"]) < 1e-15


def test_overlap_is_the_acceptance_rate():
    """The verification oracle accepts position 0 with the overlap as its frequency."""
    rng = np.random.default_rng(52)
    V, N = 6, 200_000
    zt = rng.normal(0, 1, V)
    zd = zt + rng.normal(0, 0.8, V)
    pd = _softmax(zd)
    c = overlap_mass(zt[None, None, :], zd[None, None, :])["overlap"][0, 0]
    target = np.broadcast_to(np.stack([zt, zt])[None], (N, 2, V))
    draft = np.broadcast_to(zd[None, None, :], (N, 1, V))
    toks = rng.choice(V, size=(N, 1), p=pd)
    seeds = rng.integers(0, 2**63, N).astype(np.uint64)
    out = oracle.verify(target, draft, toks, seed=seeds)
    freq = (out["num_accepted"] == 1).mean()
    assert abs(freq - c) < 5 * math.sqrt(c * (1 - c) / N)


def test_edge_cases():
    V = 8
    z = np.random.default_rng(53).normal(0, 2, (2, 3, V))
    # identical distributions overlap fully
    assert np.allclose(overlap_mass(z, z[:, :2])["overlap"], 1.0, rtol=0, atol=1e-14)
    # disjoint top-k supports do not overlap at all
    t = np.zeros((1, 2, V)); d = np.zeros((1, 1, V))
    t[0, 0, :2] = 5.0
    d[0, 0, 5:7] = 5.0
    out = overlap_mass(t, d, top_k=np.array([2]))
    assert out["overlap"][0, 0] == 0.0 and out["status"][0] == 0
    # beyond the verify length, greedy requests and bad data give NaN
    L = np.array([1, 2])
    c = overlap_mass(z, z[:, :2] + 1.0, lengths=L)["overlap"]
    assert np.isfinite(c[0, 0]) and np.isnan(c[0, 1]) and np.isfinite(c[1]).all()
    g = overlap_mass(z, z[:, :2], temperature=np.array([0.0, 1.0]))
    assert np.isnan(g["overlap"][0]).all() and g["status"][0] == 0
    bad = z.copy()
    bad[1, 1, 0] = np.nan
    b = overlap_mass(bad, bad[:, :2])
    assert b["status"][1] == oracle.STATUS_NONFINITE and np.isnan(b["overlap"][1]).all()
    assert overlap_mass(z, z[:, :2], lengths=np.array([3, 0]))["status"][0] == oracle.STATUS_BAD_LENGTH
