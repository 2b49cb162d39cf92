"""Oracle: Sequential Temperature Scaling of the confidence head (fp64, CPU).

Test infrastructure only (see the package docstring).

DSpark paper, §3.2.1 (post-hoc calibration) and §4.3.3 (the reliability
diagram and the ECE it reports).  The confidence head gives per-position
conditional survival probabilities c_k = sigmoid(t_k) (Eq. 7, t_k its logit);
the joint probability that the prefix through k survives is the product
a_k = c_1 ... c_k.  STS fits one temperature per position, left to right:
position k takes the grid value tau that minimises the Expected Calibration
Error of a_k on held-out data, with the temperatures of positions 1 .. k-1
already fixed.  Temperature scaling divides the logit: c_k(tau) =
sigmoid(t_k / tau), which keeps the order of the scores.

Readings (the pages give no more detail; all listed in the design notes):
  * ECE (Naeini et al., 2015, as cited): equal-width bins over [0, 1]; a value
    a falls in bin min(floor(a * bins), bins - 1); ECE = sum over bins of
    (n_b / N) |mean(y) - mean(a)| = (1 / N) sum_b |sum_{n in b} (a_n - y_n)|,
    with 15 bins by default;
  * the label of instance n at position k is y_{n,k} = 1 when draft positions
    1 .. k were all accepted (the event a_k predicts), else 0;
  * the grid of temperatures is an input; ties go to the first grid value;
  * a NaN logit makes its position's ECE values NaN; a position whose ECE
    values are all NaN gets tau = NaN (NaN never wins the minimum).
"""

import numpy as np

DEFAULT_BINS = 15


def sigmoid(x):
    """1 / (1 + exp(-x)) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def ece(a, y, bins=DEFAULT_BINS):
    """Expected Calibration Error of predictions a in [0, 1] against 0/1 outcomes y (see the
    module docstring); NaN when any prediction is NaN."""
    a = np.asarray(a, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(a).any():
        return np.nan
    b = np.minimum(np.floor(a * bins), bins - 1).astype(np.int64)
    s = np.bincount(b, weights=a - y, minlength=bins)      # per-bin sums of (a - y)
    return float(np.abs(s).sum() / len(a))


def sts_fit(conf_logits, labels, taus, bins=DEFAULT_BINS):
    """Fit per-position temperatures.

    conf_logits [N, G] (the confidence head's logits t); labels [N, G] (nonzero = the prefix
    through position k survived); taus [T] the grid.  Returns dict(tau [G], index [G] (grid index,
    -1 for NaN), ece [G, T] (the ECE of a_k at every grid value), gap [G] (second-best minus best
    ECE; the comparison margin of the choice), ece_raw [G] (ECE of the uncalibrated a_k),
    ece_fit [G] (ECE of the calibrated a_k)).
    """
    t = np.asarray(conf_logits, dtype=np.float64)
    y = (np.asarray(labels) != 0).astype(np.float64)
    taus = np.asarray(taus, dtype=np.float64)
    N, G = t.shape
    T = len(taus)
    a_prev = np.ones(N)
    raw_prev = np.ones(N)
    tau = np.full(G, np.nan)
    idx = np.full(G, -1, dtype=np.int64)
    curves = np.full((G, T), np.nan)
    gap = np.full(G, np.inf)
    ece_raw = np.zeros(G)
    ece_fit = np.zeros(G)
    for k in range(G):
        for g in range(T):
            curves[k, g] = ece(a_prev * sigmoid(t[:, k] / taus[g]), y[:, k], bins)
        c = curves[k]
        ok = ~np.isnan(c)
        if ok.any():
            g = int(np.flatnonzero(c == np.nanmin(c))[0])
            idx[k], tau[k] = g, taus[g]
            rest = np.delete(c[ok], np.flatnonzero(np.flatnonzero(ok) == g))
            gap[k] = float(rest.min() - c[g]) if len(rest) else np.inf
        a_prev = a_prev * sigmoid(t[:, k] / tau[k])
        raw_prev = raw_prev * sigmoid(t[:, k])
        ece_raw[k] = ece(raw_prev, y[:, k], bins)
        ece_fit[k] = ece(a_prev, y[:, k], bins)
    return dict(tau=tau, index=idx, ece=curves, gap=gap, ece_raw=ece_raw, ece_fit=ece_fit)


def sts_apply(conf_logits, tau):
    """Calibrated confidences sigmoid(t_k / tau_k) (fp64)."""
    t = np.asarray(conf_logits, dtype=np.float64)
    return sigmoid(t / np.asarray(tau, dtype=np.float64)[None, :])
