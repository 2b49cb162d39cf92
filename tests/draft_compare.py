"""Comparison aid for the draft sampler's GPU parity tests (not part of the oracle).

The oracle evaluates each draft logit z = U_k + W1[x_{k-1}] W2 exactly and rounds it once to the
storage type.  The GPU accumulates the product in fp32 on the matrix cores (bf16 operands), so
where the exact value lies within the fp32 accumulation bound of a rounding boundary, either
neighbouring stored value is a correct result.  For such elements `rounding_ranges` gives the
range of stored values the GPU may hold (near zero, where U and the bias cancel, it can span
several values).  A draw is then exempt from exact comparison when the weight those elements
could move reaches its CDF margin (`draw_exempt`); an argmax when they could change it.

The bound per element is (r + 2) u (sum_j |W1[x, j] W2t[v, j]| + |U_v|), u the unit roundoff of
the accumulation (2^-23 for fp32): r products and additions plus the addition of U and the final
rounding, each within u of the exact value.
"""

import numpy as np

from oracle.drafting import round_store
from oracle.verification import FLAG_EMIT_WINDOW

FP32_UNIT = 2.0 ** -23


def rounding_ranges(U_row, W1, W2t, prev, store, unit=FP32_UNIT, absW2t=None):
    """(zlo, zhi, amb) for one row: the stored values of z - e and z + e, and the elements where
    they differ (U_row [V], W1 and W2t [V, r] fp64, prev = x_{k-1}; absW2t = |W2t| when the
    caller keeps it)."""
    r = W1.shape[1]
    a = W1[prev]
    if absW2t is None:
        absW2t = np.abs(W2t)
    with np.errstate(all="ignore"):
        zx = U_row + W2t @ a
        e = (r + 2) * unit * (absW2t @ np.abs(a) + np.abs(U_row))
    zlo, zhi = round_store(zx - e, store), round_store(zx + e, store)
    return zlo, zhi, zlo != zhi


def greedy_ambiguous(z, zlo, zhi, amb):
    """True when some choice of values within the ambiguous elements' ranges could move the
    first-occurrence argmax of z."""
    if not amb.any():
        return False
    top = int(np.argmax(z))
    hi = np.where(amb, zhi, z)
    lo_top = zlo[top] if amb[top] else z[top]
    others = hi.copy()
    others[top] = -np.inf
    best = others.max()
    if lo_top > best:
        return False
    if lo_top < best:
        return True
    return bool(np.any(np.nonzero(others == best)[0] < top))


def draw_exempt(z, zlo, zhi, amb, T, margin):
    """Whether the draw from stored row z (temperature T, the oracle's CDF margin / W) may differ
    from the oracle's because of the ambiguous elements."""
    if T == 0.0:
        return greedy_ambiguous(z, zlo, zhi, amb)
    y = z / T
    ymax = np.max(y)
    W = np.exp(y - ymax).sum()
    window = FLAG_EMIT_WINDOW * W
    if amb.any():
        window += 2.0 * (np.exp(zhi[amb] / T - ymax) - np.exp(zlo[amb] / T - ymax)).sum()
    return margin * W < window
