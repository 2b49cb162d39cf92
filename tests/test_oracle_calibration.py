"""Pins of the Sequential Temperature Scaling oracle (DSpark paper, §3.2.1, post-hoc calibration)."""

import numpy as np
from sklearn.calibration import calibration_curve

from oracle.calibration import ece, sigmoid, sts_apply, sts_fit


def _ece_sklearn(a, y, bins):
    """ECE from scikit-learn's reliability curve (uniform bins) weighted by the bin counts."""
    prob_true, prob_pred = calibration_curve(y, a, n_bins=bins, strategy="uniform")
    counts = np.histogram(a, bins=np.linspace(0.0, 1.0, bins + 1))[0]
    counts = counts[counts > 0]
    return float((counts / len(a) * np.abs(prob_true - prob_pred)).sum())


def _synthetic(N, G, kappa, seed):
    """True conditional survival sigmoid(eta); the head's logits are kappa_k * eta (overconfident
    for kappa > 1); labels: the prefix through k survives."""
    rng = np.random.default_rng(seed)
    eta = rng.normal(1.5, 1.5, (N, G))
    acc = rng.random((N, G)) < sigmoid(eta)
    y = np.cumprod(acc, axis=1).astype(np.uint8)
    return kappa[None, :] * eta, y


def test_ece_matches_scikit_learn():
    rng = np.random.default_rng(1)
    for bins in (10, 15, 20):
        a = rng.random(5000) ** 1.5
        y = (rng.random(5000) < a ** 0.8).astype(np.float64)
        assert abs(ece(a, y, bins) - _ece_sklearn(a, y, bins)) < 1e-12


def test_ece_closed_forms():
    # all predictions in one bin: |mean(a) - mean(y)|
    a = np.full(100, 0.71)
    y = np.r_[np.ones(60), np.zeros(40)]
    assert abs(ece(a, y) - 0.11) < 1e-15
    # calibrated by construction: predictions equal to the outcome frequencies of their bin
    rng = np.random.default_rng(2)
    a = rng.random(400000)
    y = rng.random(400000) < a
    assert ece(a, y) < 0.005
    assert np.isnan(ece(np.array([0.2, np.nan]), np.array([0, 1])))


def test_recovers_the_temperature_of_an_overconfident_head():
    """Logits scaled by kappa_k are calibrated exactly at tau_k = kappa_k: the fit lands within
    a few grid steps of it and lowers the ECE well below the raw one."""
    kappa = np.array([2.0, 1.5, 3.0, 0.7])
    t, y = _synthetic(200000, 4, kappa, 3)
    taus = np.exp(np.linspace(np.log(0.25), np.log(8.0), 121))
    fit = sts_fit(t, y, taus)
    assert np.all(np.abs(np.log(fit["tau"]) - np.log(kappa)) < 0.12), fit["tau"]
    assert np.all(fit["ece_fit"] < 0.01)
    assert np.all(fit["ece_raw"][[0, 2]] > 0.03)


def test_left_to_right_and_order_preserving():
    kappa = np.array([1.8, 2.5, 1.2])
    t, y = _synthetic(20000, 3, kappa, 4)
    taus = np.exp(np.linspace(np.log(0.5), np.log(4.0), 41))
    full = sts_fit(t, y, taus)
    head = sts_fit(t[:, :2], y[:, :2], taus)
    assert np.array_equal(full["tau"][:2], head["tau"])          # later positions do not matter
    c = sts_apply(t, full["tau"])
    for k in range(3):
        assert np.array_equal(np.argsort(t[:, k], kind="stable"), np.argsort(c[:, k], kind="stable"))


def test_grid_choice_by_an_independent_ece():
    """Position 1 by exhaustion with the scikit-learn ECE: the same grid value wins."""
    t, y = _synthetic(3000, 1, np.array([2.2]), 5)
    taus = np.exp(np.linspace(np.log(0.5), np.log(5.0), 30))
    fit = sts_fit(t, y, taus)
    e = [_ece_sklearn(sigmoid(t[:, 0] / tau), y[:, 0].astype(float), 15) for tau in taus]
    assert fit["index"][0] == int(np.argmin(e))
    assert np.allclose(fit["ece"][0], e, rtol=0, atol=1e-12)
    # tau = 1 is in no grid here; with it in the grid the fit can only improve on the raw ECE
    taus1 = np.r_[taus, 1.0]
    fit1 = sts_fit(t, y, taus1)
    assert fit1["ece_fit"][0] <= fit1["ece_raw"][0] + 1e-15


def test_nan_logits():
    t, y = _synthetic(500, 3, np.array([2.0, 2.0, 2.0]), 6)
    t[7, 1] = np.nan
    fit = sts_fit(t, y, np.array([0.5, 1.0, 2.0]))
    assert np.isfinite(fit["tau"][0]) and np.isnan(fit["tau"][1:]).all()
    assert (fit["index"][1:] == -1).all() and np.isnan(fit["ece"][1:]).all()
