"""Oracle: confidence-scheduled verification lengths (CPU, exact arithmetic).

Test infrastructure only (see the package docstring).

Follows the DSpark paper, §3.2.2 (hardware-aware prefix scheduler), and
Algorithm 1 as printed in the paper's Chinese translation:

  * survival a_{r,j} = product of c_{r,1..j}, left to right (float32 products);
  * candidate pool E = {(r, j) : a_{r,j} > 0}, sorted by survival descending
    (ties: request ascending, then position ascending);
  * admitting the first m candidates gives batch tokens B_tok = R + m and
    expected accepted tokens tau(m) = R + (sum of the first m survivals);
    the objective is Theta(m) = tau(m) * SPS(B_tok), SPS read from a cost
    table indexed by batch tokens;
  * early-stop mode (Algorithm 1): admit in sorted order while Theta rises
    strictly; stop at the first candidate whose Theta is not above the best;
  * global mode (the search of §5.2, no break): the smallest m maximising
    Theta over the admissible range;
  * asynchronous mode (§5.2): the capacity K is the global search's admission
    count on confidences from two steps earlier; the current candidates are
    admitted in sorted order up to K (top-K, rank-preserving);
  * l_r = number of admitted candidates of request r.

Exact-arithmetic readings (so a parallel device scan can agree bit for bit):
tau is kept in fixed point with 47 fractional bits, q(a) = floor(a * 2^47) as
an exact integer; Theta(m) = float64(tau(m)) * 2^-47 * SPS[R + m], each step
an IEEE fp64 operation.  The verify budget caps B_tok <= budget, so
m <= budget - R.
"""

import math

import numpy as np

FRAC_BITS = 47   # tau <= R + R*gamma <= 2^15 tokens must fit a signed 64-bit integer
ONE = 1 << FRAC_BITS
MODE_EARLY_STOP = 0
MODE_GLOBAL = 1


def survival(conf):
    """a[r, j] = c[r, 0] * ... * c[r, j] in float32, multiplied left to right."""
    c = np.asarray(conf, dtype=np.float32)
    a = np.empty_like(c)
    if c.shape[1] == 0:
        return a
    a[:, 0] = c[:, 0]
    for j in range(1, c.shape[1]):
        a[:, j] = a[:, j - 1] * c[:, j]      # float32 * float32 -> float32 (one rounding)
    return a


def fixed_point(a):
    """q(a) = floor(a * 2^47) as an exact Python integer (a is a float32 value in [0, 1])."""
    return int(math.floor(float(a) * float(ONE)))


def candidates(a):
    """Sorted pool: list of (r, j) with a[r, j] > 0, by (a descending, r, j)."""
    R, G = a.shape
    pool = [(r, j) for r in range(R) for j in range(G) if a[r, j] > 0]
    pool.sort(key=lambda rj: (-float(a[rj[0], rj[1]]), rj[0], rj[1]))
    return pool


def theta(tau_fixed, sps_value):
    """Theta = fp64(tau) * 2^-47 * SPS, left to right."""
    return float(tau_fixed) * (2.0 ** -FRAC_BITS) * float(sps_value)


def theta_path(conf, sps, budget):
    """Theta(m) for m = 0 .. m_max along the sorted admission path, and the pool."""
    a = survival(conf)
    R = a.shape[0]
    pool = candidates(a)
    m_max = max(0, min(len(pool), int(budget) - R))
    tau = R * ONE
    path = [theta(tau, sps[R])]
    for m in range(1, m_max + 1):
        r, j = pool[m - 1]
        tau += fixed_point(a[r, j])
        path.append(theta(tau, sps[R + m]))
    return path, pool, a


def schedule(conf, sps, budget, mode=MODE_EARLY_STOP):
    """Per-request verify lengths and the Theta they reach.

    conf: [R, gamma] confidences in [0, 1]; sps: dense cost table (fp64),
    index = batch tokens, long enough for R + m_max; budget: cap on batch
    tokens.  Returns (lengths int64 [R], theta_best float).
    """
    path, pool, a = theta_path(conf, sps, budget)
    if mode == MODE_EARLY_STOP:
        best = path[0]
        m_star = 0
        for m in range(1, len(path)):
            if path[m] > best:
                best = path[m]
                m_star = m
            else:
                break
    elif mode == MODE_GLOBAL:
        m_star = 0
        best = path[0]
        for m in range(1, len(path)):
            if path[m] > best:
                best = path[m]
                m_star = m
    else:
        raise ValueError(mode)
    lengths = np.zeros(a.shape[0], dtype=np.int64)
    for r, _ in pool[:m_star]:
        lengths[r] += 1
    return lengths, best


def capacity(conf_hist, sps, budget):
    """Capacity K of the asynchronous scheduler (DSpark paper, §5.2): the number of candidates the
    global search (no early-stop break) admits on the confidences predicted two steps earlier."""
    lengths, _ = schedule(conf_hist, sps, budget, MODE_GLOBAL)
    return int(lengths.sum())


def schedule_topk(conf, K):
    """Lengths of the asynchronous scheduler (DSpark paper, §5.2): the current candidates, sorted by
    their up-to-date survival (ties: request, then position), admitted in that order up to K (the
    capacity fixed earlier) -- a rank-preserving top-K selection.  Returns lengths int64 [R]."""
    a = survival(conf)
    pool = candidates(a)
    lengths = np.zeros(a.shape[0], dtype=np.int64)
    for r, _ in pool[:max(0, int(K))]:
        lengths[r] += 1
    return lengths


def schedule_bruteforce(conf, sps, budget):
    """Global optimum over every length vector with sum(1 + l_r) <= budget (small R only).

    l_r ranges over 0 .. (number of positions of r with a > 0); tau and Theta
    use the same fixed-point and fp64 steps as `schedule`.  Returns
    (best Theta, list of every length vector reaching it).
    """
    a = survival(conf)
    R, G = a.shape
    q = [[fixed_point(a[r, j]) for j in range(G)] for r in range(R)]
    lmax = [int((a[r] > 0).sum()) for r in range(R)]
    best = -math.inf
    arg = []

    def rec(r, lens, tau, btok):
        nonlocal best, arg
        if r == R:
            if btok > budget:
                return
            th = theta(tau, sps[btok])
            if th > best:
                best, arg = th, [tuple(lens)]
            elif th == best:
                arg.append(tuple(lens))
            return
        acc = 0
        for l in range(lmax[r] + 1):
            if l > 0:
                acc += q[r][l - 1]
            rec(r + 1, lens + [l], tau + acc, btok + 1 + l)

    rec(0, [], R * ONE, 0)
    return best, arg
