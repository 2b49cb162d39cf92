"""GPU parity of Sequential Temperature Scaling (DSpark paper, §3.2.1, post-hoc calibration):
spec_sts_fit, spec_sts_apply and the confidence temperatures of spec_draft_markov, against the CPU
oracle.

Tolerances: every ECE is a sum of fp64 terms, accumulated in another order than the oracle's, so
|gpu - oracle| <= 1e-12 (the terms are below 1 in magnitude and N <= 2^20).  The chosen grid index
must equal the oracle's unless the oracle's best and second-best ECE lie within 1e-12 of each
other (then either is correct and the comparison stops at that position: later positions depend
on the choice).  Calibrated confidences are fp64 sigmoids rounded to fp32: within 1 fp32 ulp.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from parity import to_np
from workloads import make_draft_inputs, make_sts_inputs, tau_grid

DEV = "cuda:0"
ECE_TOL = 1e-12


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _compare_fit(got, ref, G):
    """Compare position by position; returns the number of positions compared."""
    for k in range(G):
        ie, ir = int(got["index"][k]), int(ref["index"][k])
        ce, cr = got["ece"][k], ref["ece"][k]
        nan_g, nan_r = np.isnan(ce), np.isnan(cr)
        assert (nan_g == nan_r).all(), k
        ok = ~nan_r
        assert np.all(np.abs(ce[ok] - cr[ok]) <= ECE_TOL), (k, np.max(np.abs(ce[ok] - cr[ok])))
        if ie != ir:
            assert ref["gap"][k] <= 2 * ECE_TOL, (k, ie, ir, ref["gap"][k])
            return k + 1
        if ir >= 0:
            assert got["tau"][k] == ref["tau"][k]
        else:
            assert np.isnan(got["tau"][k])
    return G


@pytest.mark.parametrize("N,G,ntau,bins,seed", [
    (5000, 5, 64, 15, 1),
    (3077, 3, 300, 7, 2),      # a partial chunk; two workgroup rows of grid values, one partial
    (1024, 4, 256, 32, 3),     # two whole chunks; the largest bin count
    (1, 2, 5, 15, 4),          # a single instance
])
def test_fit_matches_oracle(sv, N, G, ntau, bins, seed):
    t, y, _ = make_sts_inputs(N, G, seed, device=DEV)
    taus = tau_grid(ntau, device=DEV)
    out = sv.sts_fit(t, y, taus, bins)
    torch.cuda.synchronize()
    got = {k: to_np(v) for k, v in out.items()}
    ref = oracle.sts_fit(to_np(t), to_np(y), to_np(taus), bins)
    assert _compare_fit(got, ref, G) >= 1


def test_fit_nan_logit(sv):
    t, y, _ = make_sts_inputs(2000, 3, 5, device=DEV)
    t[17, 1] = float("nan")
    taus = tau_grid(32, device=DEV)
    out = sv.sts_fit(t, y, taus)
    torch.cuda.synchronize()
    tau, idx, e = to_np(out["tau"]), to_np(out["index"]), to_np(out["ece"])
    assert np.isfinite(tau[0]) and np.isnan(tau[1:]).all()
    assert (idx[1:] == -1).all() and np.isnan(e[1:]).all()
    ref = oracle.sts_fit(to_np(t), to_np(y), to_np(taus))
    assert idx[0] == ref["index"][0]


def test_fit_full_size_first_positions(sv):
    """N = 2^20 held-out instances, 16 positions, 256 grid values: every position is fitted on the
    GPU; the oracle checks the first two (a position depends on earlier ones only)."""
    N, G = 1 << 20, 16
    t, y, kappa = make_sts_inputs(N, G, 11, device=DEV)
    taus = tau_grid(256, device=DEV)
    out = sv.sts_fit(t, y, taus)
    torch.cuda.synchronize()
    got = {k: to_np(v) for k, v in out.items()}
    assert np.isfinite(got["tau"]).all()
    ref = oracle.sts_fit(to_np(t)[:, :2], to_np(y)[:, :2], to_np(taus))
    _compare_fit({k: v[:2] for k, v in got.items()}, ref, 2)
    # the synthetic head is overconfident by kappa_k: the fit scales it back
    assert np.all(np.abs(np.log(got["tau"]) - np.log(kappa)) < 0.25), (got["tau"], kappa)


def test_apply(sv):
    t, _, _ = make_sts_inputs(777, 6, 6, device=DEV)
    tau = torch.tensor([0.5, 1.0, 2.0, 3.5, 0.25, 8.0], dtype=torch.float64, device=DEV)
    c = to_np(sv.sts_apply(t, tau))
    ref = oracle.sts_apply(to_np(t), to_np(tau))
    assert np.all(np.abs(c - ref) <= np.spacing(np.float32(ref)))


def test_draft_confidence_temperatures(sv):
    B, G, V = 16, 4, 3001
    w = make_draft_inputs(B, G, V, 64, 32, "bf16", "grid", "mixed", 7, DEV)
    tau = torch.tensor([2.0, 0.7, 1.3, 3.0], dtype=torch.float64, device=DEV)
    out = sv.draft_markov(w.base, w.W1, w.W2t, w.anchor, w.temperature, w.seed, w.hidden, w.conf_w, conf_tau=tau)
    torch.cuda.synchronize()
    ref = oracle.markov_draft(w.base, w.W1.cpu(), w.W2t.cpu(), w.anchor.cpu(), w.temperature.cpu(), w.seed.cpu(),
                              w.hidden, w.conf_w.cpu(), conf_tau=to_np(tau))
    assert np.array_equal(to_np(out["tokens"]), ref["tokens"])
    c = to_np(out["conf"])
    assert np.all(np.abs(c - ref["conf"]) <= 2 * np.spacing(np.float32(ref["conf"])))
