"""Oracle: lossless rejection-sampling verification of draft blocks (fp64, CPU).

Test infrastructure only (see the package docstring).

What is computed, per request i with verify length L (DSpark paper, §2.1 and
§1; the appendix counterexample for L = 0):

  1. Per row, the distribution p = softmax(z / T) over the kept set.  The
     kept set is the whole vocabulary, or, with top-k = K, every v whose raw
     logit is at least the K-th largest raw logit of the row (ties kept).
     Logits are upcast exactly to fp64; y = z / T is an fp64 division;
     lse = max(y) + log(sum(exp(y - max(y)))) over the kept set.
  2. Draft position k = 0 .. L-1 in order: the draft token x_k is accepted
     iff u_acc(k) < r_k, r_k = min(1, p_t(x_k) / p_d(x_k)), computed as
     exp(log p_t(x_k) - log p_d(x_k)) in fp64 (r = 0 if p_t(x_k) = 0;
     r = 1 if p_d(x_k) = 0 < p_t(x_k)).  The first rejection ends the block.
  3. The emitted token comes from row n (n = first rejected position, or L
     when all L were accepted): weights w = max(0, p_t - p_d) at a rejection,
     w = p_t of target row L otherwise (with L = 0 this is the fresh token the
     target draws on its own).  Inverse CDF in ascending token order: the
     smallest v with C(v) > u_emit(n) * W, C the running sum, W = C[V-1].
  4. Outputs: n, the n accepted tokens then the emitted one (then -1), r_k for
     every k < L (NaN beyond), and a status word for bad data.
  Greedy rule (T = 0): a_k = first-occurrence argmax of raw target row k;
  n = first k < L with x_k != a_k (else L); emit a_n; r_k = [x_k == a_k].

Readings where the pages are silent (all listed in the design notes): the
residual rule max(0, p_t - p_d) is the standard correction of the method the
paper builds on; temperature divides both target and draft logits; T = 0 is
the greedy rule; ties in the inverse CDF resolve to the lower token id; the
generator is Philox4x64-10 with the counter layout documented in
`oracle.philox`.

Flags: a draw is "near its threshold" when |u_acc - r| < 1e-6 for an
acceptance test that was actually made (k <= n), or when u_emit * W lies
within 1e-10 * W of either end of the chosen CDF interval.  Flagged requests
are exempt from bit-exact comparison and are counted.

The work is vectorised over a chunk of requests (plain numpy array
operations, the same steps in the same order); chunks bound the memory.
"""

import numpy as np

from .philox import uniforms

STATUS_BAD_TOKEN = 1
STATUS_BAD_TEMPERATURE = 2
STATUS_NONFINITE = 4
STATUS_BAD_LENGTH = 8
STATUS_BAD_TOPK = 16

FLAG_ACCEPT_WINDOW = 1e-6
FLAG_EMIT_WINDOW = 1e-10

_CHUNK_ELEMS = 1 << 24


def _as_np(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()          # exact: every bf16 value is an fp32 value
        a = a.numpy()
    return np.asarray(a)


def kept_mask(z, top_k):
    """Kept set of rows z[..., V]: all v, or z_v >= the K-th largest z of the row (ties kept).

    top_k broadcasts against z.shape[:-1]; K <= 0 or K >= V keeps everything.
    """
    z = np.asarray(z)
    V = z.shape[-1]
    K = np.broadcast_to(np.asarray(top_k, dtype=np.int64), z.shape[:-1])
    keep = np.ones(z.shape, dtype=bool)
    for kv in np.unique(K):
        kv = int(kv)
        if kv <= 0 or kv >= V:
            continue
        sel = K == kv
        rows = z[sel]
        kth = np.partition(rows, V - kv, axis=-1)[..., V - kv]   # K-th largest, with multiplicity
        keep[sel] = rows >= kth[..., None]
    return keep


def log_probs(z, T, top_k=0):
    """log softmax(z / T) over the kept set of each row of z[..., V], fp64; -inf outside it.

    T broadcasts against z.shape[:-1] and must be > 0.
    """
    z = np.asarray(z).astype(np.float64)
    keep = kept_mask(z, top_k)
    T = np.asarray(T, dtype=np.float64)[..., None]
    y = z / T
    ym = np.where(keep, y, -np.inf)
    m = np.max(ym, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.where(keep, np.exp(ym - m), 0.0)
    lse = m + np.log(np.sum(e, axis=-1, keepdims=True))
    return np.where(keep, y - lse, -np.inf)


def inverse_cdf(w, u):
    """Inverse CDF of non-negative weights w[b, V] in ascending token order at u[b] in [0, 1).

    Token = smallest v with C(v) > u * W, C the running sum, W = C[V-1]; a
    target past the end (rounding) resolves to the last v with w > 0.
    Returns (token [b], W [b], flagged [b]): flagged when u * W lies within
    1e-10 * W of either end of the chosen interval [C(v-1), C(v)).
    """
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    b, V = w.shape
    ar = np.arange(b)
    C = np.cumsum(w, axis=1)
    W = C[:, -1]
    target = u * W
    tk = (C <= target[:, None]).sum(axis=1)
    past = tk >= V
    if past.any():
        tk[past] = V - 1 - np.argmax((w[past] > 0)[:, ::-1], axis=1)
    lo = np.where(tk > 0, C[ar, np.maximum(tk - 1, 0)], 0.0)
    hi = C[ar, tk]
    flagged = ((target - lo) < FLAG_EMIT_WINDOW * W) | ((hi - target) < FLAG_EMIT_WINDOW * W)
    return tk, W, flagged


def _bad_rows(z):
    """True for rows (last axis) holding a NaN or a +inf, or no finite logit at all (every kept
    set contains the row's maximum, so such a row has no finite logit in its kept set either)."""
    return np.isnan(z).any(axis=-1) | np.isposinf(z).any(axis=-1) | ~np.isfinite(z).any(axis=-1)


def _verify_chunk(i0, tgt, drf, tok, L, T, K, S):
    """Verify requests i0 .. i0+b-1 (b = len(L)); arrays already numpy, per chunk."""
    b, G1, V = tgt.shape
    G = G1 - 1
    kk = np.arange(G1)
    ridx = np.arange(b) + i0

    # ---- status (bad data never reaches the arithmetic) ----
    st = np.zeros(b, dtype=np.int64)
    badlen = (L < 0) | (L > G)
    st[badlen] = STATUS_BAD_LENGTH
    Lc = np.where(badlen, 0, L)
    st |= np.where(~(np.isfinite(T) & (T >= 0.0)), STATUS_BAD_TEMPERATURE, 0) * ~badlen
    st |= np.where(K < 0, STATUS_BAD_TOPK, 0) * ~badlen
    need_d = kk[None, :G] < Lc[:, None]                                  # [b, G]
    badtok = ((tok < 0) | (tok >= V)) & need_d
    st |= np.where(badtok.any(axis=1), STATUS_BAD_TOKEN, 0) * ~badlen
    need_t = kk[None, :] <= Lc[:, None]                                  # [b, G+1]
    bad_t = (_bad_rows(tgt) & need_t).any(axis=1)
    greedy = T == 0.0
    bad_d = np.zeros(b, dtype=bool) if drf is None else (_bad_rows(drf) & need_d).any(axis=1) & ~greedy
    st |= np.where(bad_t | bad_d, STATUS_NONFINITE, 0) * ~badlen
    ok = st == 0

    n = np.zeros(b, dtype=np.int64)
    out_tok = np.full((b, G1), -1, dtype=np.int64)
    r = np.full((b, G), np.nan)
    aflags = np.zeros(b, dtype=np.int64)
    eflag = np.zeros(b, dtype=bool)
    draws = np.zeros(b, dtype=np.int64)
    xs = np.where(need_d & ok[:, None], tok, 0)

    # ---- greedy requests: first-occurrence argmax of each raw target row ----
    g = ok & greedy
    if g.any():
        am = np.argmax(tgt[g], axis=-1)                                  # [bg, G+1]
        match = xs[g] == am[:, :G]
        rr = np.where(match, 1.0, 0.0)
        rr[~need_d[g]] = np.nan
        r[g] = rr
        mism = ~match & need_d[g]
        ng = np.where(mism.any(axis=1), np.argmax(mism, axis=1), Lc[g])
        n[g] = ng
        ot = np.where(kk[None, :G] < ng[:, None], xs[g], -1)
        ot = np.concatenate([ot, np.full((len(ng), 1), -1)], axis=1)
        ot[np.arange(len(ng)), ng] = am[np.arange(len(ng)), ng]
        out_tok[g] = ot

    # ---- sampling requests ----
    s = ok & ~greedy
    if s.any():
        si = np.nonzero(s)[0]
        Ts, Ks, Ls = T[si], K[si], Lc[si]
        lp_t = log_probs(tgt[si], Ts[:, None], Ks[:, None])             # [bs, G+1, V]
        lp_d = log_probs(drf[si], Ts[:, None], Ks[:, None])             # [bs, G, V]
        x = xs[si]
        ar = np.arange(len(si))
        a = np.take_along_axis(lp_t[:, :G], x[..., None], axis=-1)[..., 0]
        bb = np.take_along_axis(lp_d, x[..., None], axis=-1)[..., 0]
        with np.errstate(over="ignore", invalid="ignore"):
            rr = np.minimum(1.0, np.exp(a - bb))
        rr = np.where(a == -np.inf, 0.0, np.where(bb == -np.inf, 1.0, rr))
        nd = need_d[si]
        rr[~nd] = np.nan
        r[si] = rr
        u_acc, u_res = uniforms(S[si][:, None], ridx[si][:, None], kk[None, :])   # [bs, G+1]
        rej = nd & ~(u_acc[:, :G] < rr)
        ns = np.where(rej.any(axis=1), np.argmax(rej, axis=1), Ls)
        n[si] = ns
        tested = nd & (kk[None, :G] <= ns[:, None])
        aflags[si] = (tested & (np.abs(u_acc[:, :G] - rr) < FLAG_ACCEPT_WINDOW)).sum(axis=1)
        draws[si] = tested.sum(axis=1) + 1

        # emit weights on row n: residual after a rejection, target row L otherwise
        p_t = np.exp(lp_t[ar, ns])                                       # [bs, V]
        at_rej = ns < Ls
        p_d = np.exp(lp_d[ar, np.minimum(ns, G - 1)]) if G > 0 else np.zeros_like(p_t)
        w = np.where(at_rej[:, None], np.maximum(0.0, p_t - p_d), p_t)
        empty = ~(w.sum(axis=1) > 0.0)
        w[empty] = p_t[empty]
        tk, _, eflag[si] = inverse_cdf(w, u_res[ar, ns])
        ot = np.where(kk[None, :G] < ns[:, None], x, -1)
        ot = np.concatenate([ot, np.full((len(si), 1), -1)], axis=1)
        ot[ar, ns] = tk
        out_tok[si] = ot
    return dict(num_accepted=n, out_tokens=out_tok, accept_prob=r, status=st,
                accept_flags=aflags, emit_flag=eflag, draws=draws)


def verify(target, draft, draft_tokens, lengths=None, temperature=None, top_k=None, seed=None,
           requests=None):
    """Verify a batch.  Arrays may be numpy or torch (bf16 is upcast exactly).

    target [B, G+1, V]; draft [B, G, V] or None (greedy only); draft_tokens
    [B, G]; lengths [B] or None (= G); temperature [B] (default 1); top_k [B]
    or None; seed [B] uint64 bit patterns (default 0).  `requests` restricts
    the work to a subset of request indices; the others keep num_accepted 0
    and out_tokens -1.  Returns a dict of numpy arrays indexed by request.
    """
    B, G1, V = target.shape
    G = G1 - 1
    tok = _as_np(draft_tokens).astype(np.int64).reshape(B, G)
    Ls = np.full(B, G, dtype=np.int64) if lengths is None else _as_np(lengths).astype(np.int64)
    Ts = np.ones(B) if temperature is None else _as_np(temperature).astype(np.float64)
    Ks = np.zeros(B, dtype=np.int64) if top_k is None else _as_np(top_k).astype(np.int64)
    if seed is None:
        Ss = np.zeros(B, dtype=np.uint64)
    else:
        s = _as_np(seed)
        Ss = s.view(np.uint64) if s.dtype == np.int64 else s.astype(np.uint64)
    out = dict(num_accepted=np.zeros(B, dtype=np.int64), out_tokens=np.full((B, G1), -1, dtype=np.int64),
               accept_prob=np.full((B, G), np.nan), status=np.zeros(B, dtype=np.int64),
               accept_flags=np.zeros(B, dtype=np.int64), emit_flag=np.zeros(B, dtype=bool),
               draws=np.zeros(B, dtype=np.int64))
    idx = np.arange(B) if requests is None else np.asarray(sorted(set(int(i) for i in requests)))
    per = max(1, _CHUNK_ELEMS // max(1, (2 * G + 1) * V))
    pos = 0
    while pos < len(idx):
        # a chunk is a run of consecutive request indices (Philox counters carry the index)
        j = pos
        while j + 1 < len(idx) and j + 1 - pos < per and idx[j + 1] == idx[j] + 1:
            j += 1
        i0, i1 = int(idx[pos]), int(idx[j]) + 1
        tgt = _as_np(target[i0:i1]).astype(np.float64)
        drf = None if draft is None else _as_np(draft[i0:i1]).astype(np.float64)
        if drf is None and (Ts[i0:i1] != 0).any():
            raise ValueError("draft logits are required for requests with temperature != 0")
        with np.errstate(all="ignore"):
            res = _verify_chunk(i0, tgt, drf, tok[i0:i1], Ls[i0:i1], Ts[i0:i1], Ks[i0:i1],
                                Ss[i0:i1])
        for key, val in res.items():
            out[key][i0:i1] = val
        pos = j + 1
    return out


def verify_greedy(target, draft_tokens, lengths=None, requests=None):
    """Greedy verification of a batch: the greedy rule for every request."""
    B = target.shape[0]
    return verify(target, None, draft_tokens, lengths, np.zeros(B), None, None, requests)


def verify_left_to_right(target, draft, draft_tokens, lengths=None, temperature=None, top_k=None, seed=None,
                         requests=None):
    """Verification as a walk over the draft positions that stops at the first rejection.

    DSpark paper, §2.1: positions are verified left to right, and the first rejection discards
    every later draft token whatever it is, so nothing after it is examined.  This function
    takes those steps one request and one position at a time:

      for k = 0 .. L-1: target row k and draft row k are examined (a row with a NaN, a +inf or
        no finite logit ends the walk with STATUS_NONFINITE); r_k is computed and tested
        against u_acc(k) as in `verify`; a rejection ends the walk with n = k and the token
        drawn from the residual of row pair k;
      if all L drafts pass, target row L is examined and the token drawn from it.

    Everything `verify` computes for the positions the walk reaches is the same (one row at a
    time through the same `log_probs`, `uniforms` and `inverse_cdf`).  What differs is what the
    walk never reaches: accept_prob is NaN for k > n, and a bad row after the first rejection
    does not set STATUS_NONFINITE.  The argument checks (length, temperature, top-k and the draft
    tokens of every k < L) are made up front, as in `verify`.  Greedy requests (T = 0) walk the
    same way with r_k = [x_k == first-occurrence argmax of target row k].
    """
    B, G1, V = target.shape
    G = G1 - 1
    tok = _as_np(draft_tokens).astype(np.int64).reshape(B, G)
    Ls = np.full(B, G, dtype=np.int64) if lengths is None else _as_np(lengths).astype(np.int64)
    Ts = np.ones(B) if temperature is None else _as_np(temperature).astype(np.float64)
    Ks = np.zeros(B, dtype=np.int64) if top_k is None else _as_np(top_k).astype(np.int64)
    if seed is None:
        Ss = np.zeros(B, dtype=np.uint64)
    else:
        s = _as_np(seed)
        Ss = s.view(np.uint64) if s.dtype == np.int64 else s.astype(np.uint64)
    out = dict(num_accepted=np.zeros(B, dtype=np.int64), out_tokens=np.full((B, G1), -1, dtype=np.int64),
               accept_prob=np.full((B, G), np.nan), status=np.zeros(B, dtype=np.int64),
               accept_flags=np.zeros(B, dtype=np.int64), emit_flag=np.zeros(B, dtype=bool),
               draws=np.zeros(B, dtype=np.int64))
    idx = range(B) if requests is None else sorted(set(int(i) for i in requests))
    with np.errstate(all="ignore"):
        for i in idx:
            _walk_request(i, target, draft, tok[i], int(Ls[i]), float(Ts[i]), int(Ks[i]), Ss[i], V, G, out)
    return out


def _walk_request(i, target, draft, x, L, T, K, seed, V, G, out):
    """One request of `verify_left_to_right`; writes its entries of `out`."""
    # argument checks, made before anything is read (as in `verify`)
    if L < 0 or L > G:
        out["status"][i] = STATUS_BAD_LENGTH
        return
    st = 0
    if not (np.isfinite(T) and T >= 0.0):
        st |= STATUS_BAD_TEMPERATURE
    if K < 0:
        st |= STATUS_BAD_TOPK
    if ((x[:L] < 0) | (x[:L] >= V)).any():
        st |= STATUS_BAD_TOKEN
    if st:
        out["status"][i] = st
        return
    greedy = T == 0.0
    if not greedy and draft is None:
        raise ValueError("draft logits are required for requests with temperature != 0")

    def row(a, k):
        return _as_np(a[i, k]).astype(np.float64)

    tokens = out["out_tokens"][i]
    tested = 0
    for k in range(L):
        zt = row(target, k)
        zd = None if greedy else row(draft, k)
        if _bad_rows(zt) or (zd is not None and _bad_rows(zd)):
            out["status"][i] = STATUS_NONFINITE
            out["accept_prob"][i] = np.nan
            tokens[:] = -1
            return
        if greedy:
            a_k = int(np.argmax(zt))
            out["accept_prob"][i, k] = 1.0 if x[k] == a_k else 0.0
            if x[k] != a_k:
                out["num_accepted"][i] = k
                tokens[k] = a_k
                return
            tokens[k] = x[k]
            continue
        lp_t = log_probs(zt[None], np.array([T]), np.array([K]))[0]
        lp_d = log_probs(zd[None], np.array([T]), np.array([K]))[0]
        a, b = lp_t[x[k]], lp_d[x[k]]
        r = 0.0 if a == -np.inf else (1.0 if b == -np.inf else min(1.0, float(np.exp(a - b))))
        out["accept_prob"][i, k] = r
        u_acc, u_emit = uniforms(np.array([seed]), np.array([i]), np.array([k]))
        tested += 1
        out["accept_flags"][i] += int(abs(u_acc[0] - r) < FLAG_ACCEPT_WINDOW)
        if not (u_acc[0] < r):
            # rejected: the residual of row pair k
            p_t, p_d = np.exp(lp_t), np.exp(lp_d)
            w = np.maximum(0.0, p_t - p_d)
            if not (w.sum() > 0.0):
                w = p_t
            t, _, flag = inverse_cdf(w[None], u_emit)
            out["num_accepted"][i] = k
            tokens[k] = int(t[0])
            out["emit_flag"][i] = bool(flag[0])
            out["draws"][i] = tested + 1
            return
        tokens[k] = x[k]
    # every draft passed: target row L gives the appended token
    zt = row(target, L)
    if _bad_rows(zt):
        out["status"][i] = STATUS_NONFINITE
        out["accept_prob"][i] = np.nan
        tokens[:] = -1
        return
    out["num_accepted"][i] = L
    if greedy:
        tokens[L] = int(np.argmax(zt))
        return
    p_t = np.exp(log_probs(zt[None], np.array([T]), np.array([K]))[0])
    _, u_emit = uniforms(np.array([seed]), np.array([i]), np.array([L]))
    t, _, flag = inverse_cdf(p_t[None], u_emit)
    tokens[L] = int(t[0])
    out["emit_flag"][i] = bool(flag[0])
    out["draws"][i] = tested + 1
