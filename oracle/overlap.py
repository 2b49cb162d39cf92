"""Oracle: per-position overlap mass c*_k = sum_v min(p_t,k(v), p_d,k(v)) (fp64, CPU).

Test infrastructure only (see the package docstring).

DSpark paper, §3.2.1, Eq. 8: the probability that draft position k is
accepted given that it is reached equals the overlap of the target and draft
distributions at that position, sum_v min(p_t, p_d) (equivalently
1 - (1/2) * ||p_t - p_d||_1); it is the label the confidence head is trained
on and the per-position factor of the expected accepted length.

The distributions are those of the verification oracle (`log_probs`: softmax
of z / T over the kept set, fp64).  Per request i and draft position k < L_i
the output is sum_v exp(min(log p_t(v), log p_d(v))), summed in fp64; NaN for
k >= L_i, for greedy requests (T = 0: no draft distribution is involved) and
for requests with bad data.  Status words as in `verify`, without the token
check (no draft tokens are involved).
"""

import numpy as np

from .verification import (
    STATUS_BAD_LENGTH,
    STATUS_BAD_TEMPERATURE,
    STATUS_BAD_TOPK,
    STATUS_NONFINITE,
    _as_np,
    _bad_rows,
    log_probs,
)


def overlap_mass(target, draft, lengths=None, temperature=None, top_k=None):
    """c*[B, G] and status[B] (see the module docstring).

    target [B, G+1, V] (row G is not used) or [B, G, V]; draft [B, G, V];
    lengths [B] or None (= G); temperature [B] (default 1); top_k [B] or None.
    """
    B, G = draft.shape[0], draft.shape[1]
    Ls = np.full(B, G, dtype=np.int64) if lengths is None else _as_np(lengths).astype(np.int64)
    Ts = np.ones(B) if temperature is None else _as_np(temperature).astype(np.float64)
    Ks = np.zeros(B, dtype=np.int64) if top_k is None else _as_np(top_k).astype(np.int64)
    out = np.full((B, G), np.nan)
    status = np.zeros(B, dtype=np.int64)
    for i in range(B):
        L, T, K = int(Ls[i]), float(Ts[i]), int(Ks[i])
        if L < 0 or L > G:
            status[i] = STATUS_BAD_LENGTH
            continue
        st = 0
        if not (np.isfinite(T) and T >= 0.0):
            st |= STATUS_BAD_TEMPERATURE
        if K < 0:
            st |= STATUS_BAD_TOPK
        if st == 0 and L > 0 and T > 0.0:
            zt = _as_np(target[i, :L]).astype(np.float64)
            zd = _as_np(draft[i, :L]).astype(np.float64)
            if (_bad_rows(zt) | _bad_rows(zd)).any():
                st |= STATUS_NONFINITE
            else:
                lp_t = log_probs(zt, T, K)
                lp_d = log_probs(zd, T, K)
                out[i, :L] = np.exp(np.minimum(lp_t, lp_d)).sum(axis=-1)
        status[i] = st
        if st:
            out[i] = np.nan
    return dict(overlap=out, status=status)
