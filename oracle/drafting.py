"""Oracle: the Markov-head sequential draft sampler and the confidence head (fp64, CPU).

Test infrastructure only (see the package docstring).

DSpark paper, §3.1 (sequential stage: the block factorisation of Eq. 4 and
the Markov head of Eq. 5) and §3.2.1 (the confidence head, Eq. 7).

Per request i with anchor token x_0 (the last token of the previous
verification cycle) and base logits U_1 .. U_G from the parallel stage, for
k = 1 .. G in order:

  1. transition bias b = W1[x_{k-1}] W2 (Eq. 5): row x_{k-1} of the V x r
     embedding table times the r x V projection.  The projection is stored
     token-major, W2t [V, r] (row v = column v of W2), so b_v = sum_j
     W1[x_{k-1}, j] * W2t[v, j];
  2. draft logits z_k = U_k + b, evaluated in fp64 and rounded once to the
     storage type of the logits (bf16: round to nearest, ties to even, 8
     significant bits; fp32: numpy's conversion).  The stored row is the
     draft distribution's definition: the verifier reads it back;
  3. p_k = softmax(z_k / T) over the whole vocabulary (Eq. 4 with the
     sampling temperature); x_k = the smallest v with C(v) > u * W (C the
     running sum of exp(z / T - max) in ascending token order, W its total,
     u the draft uniform of (i, k) from `oracle.philox.draft_uniform`);
     T = 0: x_k = the first-occurrence argmax of the stored z_k;
  4. c_k = sigmoid(w . [h_k ; W1[x_{k-1}]]) (Eq. 7) when the head's weight w
     is given (with no hidden states, d = 0, the h_k part is empty); with
     per-position temperatures tau_k from Sequential Temperature Scaling
     (§3.2.1) the calibrated c_k = sigmoid(w . [...] / tau_k).

Status (request-wide, as in `verify`): bad temperature (NaN, negative,
infinite), bad token (anchor outside [0, V)), non-finite (a stored row with
a NaN or +inf, or no finite logit).  A request with a status keeps tokens -1
and confidences NaN; its logits are not defined.

Flags (as in `verify`): a draw is flagged when u * W lies within 1e-10 * W of
either end of the chosen CDF interval; `margin` reports that distance / W.
"""

import numpy as np

from .philox import draft_uniform
from .verification import (
    FLAG_EMIT_WINDOW,
    STATUS_BAD_TEMPERATURE,
    STATUS_BAD_TOKEN,
    STATUS_NONFINITE,
    _as_np,
    _bad_rows,
)

BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(z):
    """fp64 -> the nearest bf16 value (ties to even), returned as fp64.  Magnitudes that round
    above the largest finite bf16 become +-inf; bf16 subnormals are not modelled (values below
    2^-126 keep 8 significant bits)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(z)                        # z = m 2^e, 0.5 <= |m| < 1
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, z), r)
    return np.where(np.isfinite(z), r, z)


def round_store(z, store):
    if store == "bf16":
        return round_bf16(z)
    if store == "fp32":
        with np.errstate(over="ignore"):
            return np.asarray(z, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage type {store!r}")


def _inverse_cdf_margin(w, u):
    """Inverse CDF of weights w[V] at u: (token, distance of u*W to the nearer end of the chosen
    interval, W).  Past the end (rounding) resolves to the last v with w > 0."""
    C = np.cumsum(w)
    W = C[-1]
    t = u * W
    tk = int((C <= t).sum())
    if tk >= len(w):
        tk = int(np.nonzero(w > 0)[0][-1])
    lo = C[tk - 1] if tk > 0 else 0.0
    return tk, min(t - lo, C[tk] - t), W


def markov_draft(base, W1, W2t, anchor, temperature=None, seed=None, hidden=None, conf_w=None,
                 store="bf16", requests=None, conf_tau=None, first_request=0):
    """Draft G tokens per request (see the module docstring).

    base [B, G, V] (U); W1 [V, r]; W2t [V, r]; anchor [B]; temperature [B] (default 1);
    seed [B] uint64 bit patterns (default 0); hidden [B, G, d] and conf_w [d + r] (conf_w alone
    when d = 0; no confidences without conf_w); store "bf16" | "fp32".
    `requests` restricts the work to a subset (others keep status 0, tokens -1); conf_tau [G]
    the per-position temperatures of the confidences (default 1); first_request: the batch
    index of row 0 of these arrays (the draft uniform is keyed by the batch index, so a slice of
    a batch gives that batch's draws).

    Returns a dict: tokens [B, G] int64, logits [B, G, V] fp64 (stored values; NaN where not
    computed), conf [B, G], status [B], flag [B, G] bool, margin [B, G] (u*W distance / W; inf
    for greedy).
    """
    B, G, V = base.shape
    W1 = _as_np(W1).astype(np.float64)
    W2t = _as_np(W2t).astype(np.float64)
    r = W1.shape[1]
    x0 = _as_np(anchor).astype(np.int64)
    Ts = np.ones(B) if temperature is None else _as_np(temperature).astype(np.float64)
    if seed is None:
        Ss = np.zeros(B, dtype=np.uint64)
    else:
        s = _as_np(seed)
        Ss = s.view(np.uint64) if s.dtype == np.int64 else s.astype(np.uint64)
    H = None if hidden is None else hidden
    wc = None if conf_w is None else _as_np(conf_w).astype(np.float64)
    ctau = np.ones(G) if conf_tau is None else _as_np(conf_tau).astype(np.float64)
    tokens = np.full((B, G), -1, dtype=np.int64)
    logits = np.full((B, G, V), np.nan)
    conf = np.full((B, G), np.nan)
    status = np.zeros(B, dtype=np.int64)
    flag = np.zeros((B, G), dtype=bool)
    margin = np.full((B, G), np.inf)
    idx = range(B) if requests is None else sorted(set(int(i) for i in requests))
    for i in idx:
        T = Ts[i]
        st = 0
        if not (np.isfinite(T) and T >= 0.0):
            st |= STATUS_BAD_TEMPERATURE
        if not (0 <= x0[i] < V):
            st |= STATUS_BAD_TOKEN
        if st:
            status[i] = st
            continue
        U = _as_np(base[i]).astype(np.float64)
        h = None if H is None else _as_np(H[i]).astype(np.float64)
        prev = int(x0[i])
        for k in range(G):
            a = W1[prev]
            with np.errstate(all="ignore"):
                zx = U[k] + W2t @ a                                   # Eq. 5 bias added to U_k
            z = round_store(zx, store)
            logits[i, k] = z
            if _bad_rows(z[None])[0]:
                st |= STATUS_NONFINITE
                break
            if wc is not None:
                dh = len(wc) - r
                t = float(wc[dh:] @ a)                                       # Eq. 7
                if dh:
                    t += float(wc[:dh] @ h[k])
                conf[i, k] = 1.0 / (1.0 + np.exp(-t / ctau[k]))
            if T == 0.0:
                xk = int(np.argmax(z))
            else:
                y = z / T
                ymax = np.max(y)
                w = np.exp(y - ymax)
                u = float(draft_uniform(Ss[i], first_request + i, k))
                xk, mg, W = _inverse_cdf_margin(w, u)
                margin[i, k] = mg / W
                flag[i, k] = mg < FLAG_EMIT_WINDOW * W
            tokens[i, k] = xk
            prev = xk
        status[i] = st
        if st:
            tokens[i] = -1
            conf[i] = np.nan
    return dict(tokens=tokens, logits=logits, conf=conf, status=status, flag=flag, margin=margin)
