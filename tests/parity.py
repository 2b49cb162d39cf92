"""Shared GPU-vs-oracle comparison rules for the parity tests.

* num_accepted and out_tokens: bit-exact for every request whose draws are
  not flagged by the oracle (an acceptance uniform within 1e-6 of its
  threshold, or an emit target within 1e-10 * W of a CDF boundary); flagged
  requests are counted, and flagged draws must stay under 1e-4 of all draws
  on the large runs.
* accept_prob: relative error <= 1e-5 (NaN exactly where the oracle has NaN).
* status: equal.
"""

import numpy as np
import torch

import oracle

REL_TOL_PROB = 1e-5


def to_np(t):
    return t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def compare_verify(gpu, ref, requests=None, check_prob=True):
    """Compare GPU outputs with oracle outputs on `requests` (default all).

    Returns dict(compared, flagged_requests, flagged_draws, draws, mismatches).
    Raises AssertionError on any unflagged mismatch.
    """
    n_g = to_np(gpu["num_accepted"]).astype(np.int64)
    t_g = to_np(gpu["out_tokens"]).astype(np.int64)
    st_g = to_np(gpu["status"]).astype(np.int64) if gpu.get("status") is not None else None
    B = len(n_g)
    idx = np.arange(B) if requests is None else np.asarray(requests)
    flagged = ref["emit_flag"][idx] | (ref["accept_flags"][idx] > 0)
    if st_g is not None:
        bad = np.nonzero(st_g[idx] != ref["status"][idx])[0]
        assert len(bad) == 0, ("status", idx[bad][:10], st_g[idx][bad][:10], ref["status"][idx][bad][:10])
    same_n = n_g[idx] == ref["num_accepted"][idx]
    same_t = (t_g[idx] == ref["out_tokens"][idx]).all(axis=1)
    wrong = ~(same_n & same_t) & ~flagged
    if wrong.any():
        j = np.nonzero(wrong)[0][:5]
        raise AssertionError(f"unflagged mismatch at requests {idx[j].tolist()}: "
                             f"gpu n={n_g[idx][j].tolist()} ref n={ref['num_accepted'][idx][j].tolist()} "
                             f"gpu tok={t_g[idx][j].tolist()} ref tok={ref['out_tokens'][idx][j].tolist()}")
    if check_prob and gpu.get("accept_prob") is not None:
        r_g = to_np(gpu["accept_prob"]).astype(np.float64)[idx]
        r_o = ref["accept_prob"][idx]
        assert (np.isnan(r_g) == np.isnan(r_o)).all(), "NaN pattern of accept_prob differs"
        m = ~np.isnan(r_o)
        err = np.abs(r_g[m] - r_o[m])
        lim = REL_TOL_PROB * np.abs(r_o[m]) + 1e-37
        assert (err <= lim).all(), f"accept_prob rel err max {np.max(err / np.maximum(np.abs(r_o[m]), 1e-300))}"
    fd = int(ref["accept_flags"][idx].sum() + ref["emit_flag"][idx].sum())
    return dict(compared=len(idx), flagged_requests=int(flagged.sum()), flagged_draws=fd,
                draws=int(ref["draws"][idx].sum()), mismatches=int((~(same_n & same_t)).sum()))


def run_oracle(w, requests=None, lengths=None):
    L = w.lengths if lengths is None else lengths
    if w.name == "greedy" or w.draft is None:
        return oracle.verify_greedy(w.target, w.draft_tokens, L, requests=requests)
    return oracle.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed,
                         requests=requests)
