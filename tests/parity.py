"""Shared GPU-vs-oracle comparison rules for the parity tests.

* num_accepted and out_tokens: bit-exact for every request whose draws the
  oracle does not flag.  A draw is flagged when its acceptance uniform lies
  within 1e-6 of its threshold, or its emit target u * W within 1e-10 * W of a
  boundary of the chosen CDF interval (DSpark paper, §2.1 rule; the windows
  are the stated tolerance of the comparison).  A flagged request is not
  exempt: the GPU's outcome must be one the method allows when each flagged
  draw may go either way (`admissible_outcomes`).
* The count of flagged draws must stay under 1e-4 of all draws on every
  full-size run (`bound=True`).
* accept_prob: relative error <= 1e-5 (NaN exactly where the oracle has NaN).
* status: equal.

`run_oracle_pooled` runs the oracle over every request of a workload with a
pool of forked worker processes (numpy only; the workers never touch the
GPU), which is what makes whole-batch comparisons at full size affordable.
"""

import dataclasses
import os
from typing import Optional

import numpy as np
import torch

import oracle

REL_TOL_PROB = 1e-5
FLAG_BOUND = 1e-4


def to_np(t):
    return t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def _host(t, dtype=None):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()          # exact: every bf16 value is an fp32 value
        t = t.numpy()
    a = np.asarray(t)
    return a if dtype is None else a.astype(dtype)


@dataclasses.dataclass
class HostInputs:
    """Host copies of a verification batch (bf16 upcast exactly to fp32), as the oracle reads it."""
    target: np.ndarray                   # [B, G+1, V]
    draft: Optional[np.ndarray]          # [B, G, V] or None (greedy)
    tokens: np.ndarray                   # [B, G]
    lengths: np.ndarray                  # [B]
    temperature: np.ndarray              # [B]
    top_k: np.ndarray                    # [B]
    seed: np.ndarray                     # [B] uint64

    @classmethod
    def of(cls, target, draft, tokens, lengths=None, temperature=None, top_k=None, seed=None):
        t = _host(target)
        B, G1, _ = t.shape
        G = G1 - 1
        s = _host(seed)
        if s is None:
            s = np.zeros(B, dtype=np.uint64)
        elif s.dtype == np.int64:
            s = s.view(np.uint64)
        return cls(target=t, draft=_host(draft), tokens=_host(tokens, np.int64).reshape(B, G),
                   lengths=np.full(B, G, dtype=np.int64) if lengths is None else _host(lengths, np.int64),
                   temperature=np.ones(B) if temperature is None else _host(temperature, np.float64),
                   top_k=np.zeros(B, dtype=np.int64) if top_k is None else _host(top_k, np.int64),
                   seed=s.astype(np.uint64))

    @classmethod
    def of_workload(cls, w, lengths=None):
        if w.name == "greedy" or w.draft is None:
            B = w.B
            return cls.of(w.target, None, w.draft_tokens, w.lengths if lengths is None else lengths,
                          torch.zeros(B), None, None)
        return cls.of(w.target, w.draft, w.draft_tokens, w.lengths if lengths is None else lengths,
                      w.temperature, w.top_k, w.seed)


def admissible_outcomes(h: HostInputs, i: int):
    """Every (n, emitted token) the method allows for request i when each flagged draw may go
    either way: at an acceptance test whose uniform lies within 1e-6 of r both decisions, and at
    an emit draw every positive-weight token whose CDF interval comes within 1e-10 * W of the
    target u * W.  Built from the oracle's own steps (log_probs, uniforms, inverse_cdf)."""
    L = int(h.lengths[i])
    T = float(h.temperature[i])
    K = int(h.top_k[i])
    x = h.tokens[i]
    if T == 0.0:   # greedy: no draws
        am = np.argmax(h.target[i, :L + 1].astype(np.float64), axis=-1)
        mism = np.nonzero(x[:L] != am[:L])[0]
        n = int(mism[0]) if len(mism) else L
        return {(n, int(am[n]))}
    lp_t = oracle.log_probs(h.target[i, :L + 1], np.full(L + 1, T), np.full(L + 1, K))
    lp_d = oracle.log_probs(h.draft[i, :L], np.full(L, T), np.full(L, K)) if L else np.zeros((0, h.target.shape[2]))
    u_acc, u_res = oracle.uniforms(np.full(L + 1, h.seed[i], dtype=np.uint64), np.full(L + 1, i), np.arange(L + 1))
    r = np.empty(L)
    for k in range(L):
        a, b = lp_t[k, x[k]], lp_d[k, x[k]]
        r[k] = 0.0 if a == -np.inf else (1.0 if b == -np.inf else min(1.0, float(np.exp(a - b))))
    # every first-rejection position reachable when flagged tests may go either way: a flagged
    # test may reject (ending the block there) or accept (going on)
    reach = set()
    for k in range(L):
        if abs(u_acc[k] - r[k]) < oracle.FLAG_ACCEPT_WINDOW:
            reach.add(k)
        elif not (u_acc[k] < r[k]):
            reach.add(k)
            break
    else:
        reach.add(L)
    out = set()
    for n in sorted(reach):
        p_t = np.exp(lp_t[n])
        if n < L:
            w = np.maximum(0.0, p_t - np.exp(lp_d[n]))
            if not (w.sum() > 0.0):
                w = p_t
        else:
            w = p_t
        tk, W, _ = oracle.inverse_cdf(w[None], np.asarray([u_res[n]]))
        out.add((n, int(tk[0])))
        C = np.cumsum(w)
        tgt = u_res[n] * W[0]
        lo, hi = tgt - oracle.FLAG_EMIT_WINDOW * W[0], tgt + oracle.FLAG_EMIT_WINDOW * W[0]
        before = np.concatenate([[0.0], C[:-1]])
        near = np.nonzero((w > 0) & (C > lo) & (before <= hi))[0]
        out.update((n, int(v)) for v in near)
    return out


def compare_verify(gpu, ref, requests=None, check_prob=True, inputs: Optional[HostInputs] = None,
                   bound=False, left_to_right=False):
    """Compare GPU outputs with oracle outputs on `requests` (default all).

    Unflagged requests must agree bit for bit.  A flagged request that differs must have taken
    an admissible outcome (needs `inputs`; without them a flagged request is only counted).
    bound=True asserts flagged draws < 1e-4 of draws.  left_to_right: the reference is the walk that
    stops at the first rejection, whose accept_prob is NaN after it; a flagged request that stopped
    elsewhere is compared on the positions both tested.
    Returns dict(compared, flagged_requests, flagged_draws, draws, mismatches, admissible).
    """
    n_g = to_np(gpu["num_accepted"]).astype(np.int64)
    t_g = to_np(gpu["out_tokens"]).astype(np.int64)
    st_g = to_np(gpu["status"]).astype(np.int64) if gpu.get("status") is not None else None
    B = len(n_g)
    G1 = t_g.shape[1]
    idx = np.arange(B) if requests is None else np.asarray(requests)
    flagged = ref["emit_flag"][idx] | (ref["accept_flags"][idx] > 0)
    if st_g is not None:
        bad = np.nonzero(st_g[idx] != ref["status"][idx])[0]
        assert len(bad) == 0, ("status", idx[bad][:10], st_g[idx][bad][:10], ref["status"][idx][bad][:10])
    same_n = n_g[idx] == ref["num_accepted"][idx]
    same_t = (t_g[idx] == ref["out_tokens"][idx]).all(axis=1)
    differ = ~(same_n & same_t)
    wrong = differ & ~flagged
    if wrong.any():
        j = np.nonzero(wrong)[0][:5]
        raise AssertionError(f"unflagged mismatch at requests {idx[j].tolist()}: "
                             f"gpu n={n_g[idx][j].tolist()} ref n={ref['num_accepted'][idx][j].tolist()} "
                             f"gpu tok={t_g[idx][j].tolist()} ref tok={ref['out_tokens'][idx][j].tolist()}")
    admissible = 0
    if inputs is not None:
        for i in idx[differ & flagged]:
            i = int(i)
            n = int(n_g[i])
            ok = {(n, int(t_g[i, n]))} <= admissible_outcomes(inputs, i) if 0 <= n < G1 else False
            L = int(inputs.lengths[i])
            ok = ok and n <= L and (t_g[i, :n] == inputs.tokens[i, :n]).all() and (t_g[i, n + 1:] == -1).all()
            assert ok, f"request {i}: gpu (n={n}, tokens={t_g[i].tolist()}) is not an admissible outcome"
            admissible += 1
    if check_prob and gpu.get("accept_prob") is not None:
        r_g = to_np(gpu["accept_prob"]).astype(np.float64)[idx]
        r_o = ref["accept_prob"][idx]
        if left_to_right and (differ & flagged).any():
            # positions past the shorter of the two walks are left out of the comparison
            r_g, r_o = r_g.copy(), r_o.copy()
            G = r_g.shape[1]
            for j in np.nonzero(differ & flagged)[0]:
                stop = min(int(n_g[idx][j]), int(ref["num_accepted"][idx][j])) + 1
                r_g[j, stop:G] = np.nan
                r_o[j, stop:G] = np.nan
        assert (np.isnan(r_g) == np.isnan(r_o)).all(), "NaN pattern of accept_prob differs"
        m = ~np.isnan(r_o)
        err = np.abs(r_g[m] - r_o[m])
        lim = REL_TOL_PROB * np.abs(r_o[m]) + 1e-37
        assert (err <= lim).all(), f"accept_prob rel err max {np.max(err / np.maximum(np.abs(r_o[m]), 1e-300))}"
    fd = int(ref["accept_flags"][idx].sum() + ref["emit_flag"][idx].sum())
    draws = int(ref["draws"][idx].sum())
    res = dict(compared=len(idx), flagged_requests=int(flagged.sum()), flagged_draws=fd, draws=draws,
               mismatches=int(differ.sum()), admissible=admissible)
    if bound:
        assert fd < FLAG_BOUND * max(draws, 1) or fd == 0, f"flagged draws {fd} of {draws} exceed 1e-4: {res}"
    return res


def run_oracle(w, requests=None, lengths=None):
    L = w.lengths if lengths is None else lengths
    if w.name == "greedy" or w.draft is None:
        return oracle.verify_greedy(w.target, w.draft_tokens, L, requests=requests)
    return oracle.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed,
                         requests=requests)


# ---- the oracle over every request, in forked worker processes ----

_POOL_FN = {}


def _pool_task(i):
    # one BLAS thread per worker: the pool already has a process per core
    from threadpoolctl import threadpool_limits
    blk = _POOL_FN["blocks"][i]
    with threadpool_limits(1):
        return i, _POOL_FN["fn"](blk)


def pool_workers():
    """Worker processes for the pooled oracle: the host cores this process may run on, at most 16
    (the CPU share of a one-GPU machine)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool_map(fn, blocks, workers=None):
    """[fn(block) for block in blocks], computed by forked worker processes.  The workers inherit
    fn and whatever host arrays it closes over (nothing is pickled on the way in); they run numpy
    only and never touch the GPU."""
    import multiprocessing as mp
    import sys
    import time
    results = [None] * len(blocks)
    _POOL_FN.update(fn=fn, blocks=blocks)
    t0 = time.time()
    try:
        with mp.get_context("fork").Pool(workers or pool_workers()) as p:
            for done, (i, res) in enumerate(p.imap_unordered(_pool_task, range(len(blocks)), chunksize=1), 1):
                results[i] = res
                if done % max(1, len(blocks) // 4) == 0:
                    print(f"  oracle blocks {done}/{len(blocks)} in {time.time() - t0:.1f} s", flush=True)
                    sys.stdout.flush()
    finally:
        _POOL_FN.clear()
    return results


def request_blocks(B, block=4, requests=None):
    idx = np.arange(B) if requests is None else np.asarray(sorted(set(int(i) for i in requests)))
    return [idx[a:a + block].tolist() for a in range(0, len(idx), block)]


def run_oracle_pooled(h: HostInputs, requests=None, block=4, workers=None, left_to_right=False):
    """oracle.verify (oracle.verify_left_to_right with left_to_right) over `requests` (default every
    request) of the host inputs h, in blocks of consecutive requests spread over forked workers.
    Returns the oracle's dict of arrays."""
    B, G1, _ = h.target.shape
    blocks = request_blocks(B, block, requests)

    def fn(blk):
        if left_to_right:
            res = oracle.verify_left_to_right(h.target, h.draft, h.tokens, h.lengths, h.temperature, h.top_k,
                                              h.seed, requests=blk)
        elif h.draft is None:
            res = oracle.verify_greedy(h.target, h.tokens, h.lengths, requests=blk)
        else:
            res = oracle.verify(h.target, h.draft, h.tokens, h.lengths, h.temperature, h.top_k, h.seed,
                                requests=blk)
        return {k: v[blk] for k, v in res.items()}

    out = dict(num_accepted=np.zeros(B, dtype=np.int64), out_tokens=np.full((B, G1), -1, dtype=np.int64),
               accept_prob=np.full((B, G1 - 1), np.nan), status=np.zeros(B, dtype=np.int64),
               accept_flags=np.zeros(B, dtype=np.int64), emit_flag=np.zeros(B, dtype=bool),
               draws=np.zeros(B, dtype=np.int64))
    for blk, res in zip(blocks, pool_map(fn, blocks, workers)):
        for k, v in res.items():
            out[k][blk] = v
    return out
