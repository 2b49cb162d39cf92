"""GPU parity of spec_overlap_mass (the per-position overlap sum_v min(p_t, p_d), DSpark paper,
§3.2.1, Eq. 8) against the CPU oracle.

Tolerance: probabilities are fp32 (exponent formed from split float constants, hardware exp2,
about 1e-7 relative each) and summed in fp64, so |gpu - oracle| <= 1e-5 * oracle + 1e-9.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from parity import _host, pool_map, request_blocks, to_np
from workloads import make_workload

DEV = "cuda:0"
RTOL, ATOL = 1e-5, 1e-9


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _gpu(sv, w, lengths=None, temperature=None, top_k=None, target=None, draft=None):
    out = sv.overlap_mass(w.target if target is None else target, w.draft if draft is None else draft,
                          lengths, w.temperature if temperature is None else temperature,
                          w.top_k if top_k is None else top_k)
    torch.cuda.synchronize()
    return to_np(out["overlap"]), to_np(out["status"])


def _check(got, ref, st_got, st_ref):
    assert (st_got == st_ref).all(), (np.flatnonzero(st_got != st_ref)[:8], st_got, st_ref)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert (nan_g == nan_r).all(), np.argwhere(nan_g != nan_r)[:8]
    ok = ~nan_r
    err = np.abs(got[ok] - ref[ok])
    tol = RTOL * np.abs(ref[ok]) + ATOL
    assert (err <= tol).all(), (err.max(), np.argwhere(err > tol)[:4])


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(B=64, gamma=6, V=999, seed=5)),
    ("mid", dict(B=6, gamma=5, V=20011, seed=7)),
    ("mid", dict(B=4, gamma=3, V=60000, seed=8)),
    ("mixed", dict(B=12, gamma=4, V=30001, seed=9)),
    ("mixed", dict(B=8, gamma=3, V=129280, seed=12)),      # segmented top-k rows
    ("scheduled", dict(B=16, gamma=16, V=151936, seed=10)),
    ("mid", dict(B=3, gamma=8, V=524288, seed=13)),        # the largest bf16 vocabulary
    ("mid", dict(B=2, gamma=64, V=8192, seed=14)),         # the longest block
])
def test_small_all_requests(sv, name, kw):
    w = make_workload(name, DEV, **kw)
    rng = np.random.default_rng(61)
    L = torch.from_numpy(rng.integers(0, w.gamma + 1, w.B).astype(np.int32)).to(DEV)
    got, st = _gpu(sv, w, L)
    ref = oracle.overlap_mass(w.target, w.draft, L, w.temperature, w.top_k)
    _check(got, ref["overlap"], st, ref["status"])
    assert np.isfinite(got).sum() == int(to_np(L).sum())


def test_edge_cases(sv):
    w = make_workload("mid", DEV, B=8, gamma=4, V=5003, seed=62)
    t, d = w.target.clone(), w.draft.clone()
    T = w.temperature.clone()
    K = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    L = torch.full((w.B,), w.gamma, dtype=torch.int32, device=DEV)
    t[0, 1, 7] = float("nan")                  # NaN in a needed target row
    d[1, 3, 0] = float("inf")                  # +inf in a needed draft row
    d[2, 2, :] = float("-inf")                 # a needed draft row with no finite logit
    L[3] = w.gamma + 1                         # bad length
    L[4] = 0                                   # nothing to measure
    T[5] = 0.0                                 # greedy request: no draft distribution
    K[6] = 3                                   # top-k with temperature
    T[6] = 0.7
    t[7, 0] = d[7, 0]                          # identical rows overlap fully
    t[3, 4, 0] = float("nan")                  # beyond the verify length: not needed
    got, st = _gpu(sv, w, L, T, K, t, d)
    ref = oracle.overlap_mass(t, d, L, T, K)
    _check(got, ref["overlap"], st, ref["status"])
    assert abs(got[7, 0] - 1.0) < 1e-5


def test_disjoint_top_k_supports(sv):
    B, G, V = 2, 1, 4096
    t = torch.zeros((B, G + 1, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((B, G, V), dtype=torch.bfloat16, device=DEV)
    t[:, 0, :5] = 4.0
    d[:, 0, 100:105] = 4.0
    K = torch.tensor([5, 0], dtype=torch.int32, device=DEV)
    T = torch.ones(B, dtype=torch.float32, device=DEV)
    out = sv.overlap_mass(t, d, None, T, K)
    torch.cuda.synchronize()
    got = to_np(out["overlap"])
    ref = oracle.overlap_mass(t, d, None, T, K)["overlap"]
    assert got[0, 0] == 0.0 and ref[0, 0] == 0.0
    assert abs(got[1, 0] - ref[1, 0]) <= RTOL * ref[1, 0] + ATOL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["scheduled", "mixed"])
def test_full_size_all_requests(sv, name):
    """Every request of the full-size workload (the scheduled one at its scheduled lengths)
    against the oracle, in blocks of requests over forked host processes."""
    w = make_workload(name, DEV)
    if w.conf is not None:
        s = sv.schedule_lengths(w.conf, torch.from_numpy(w.sps).to(DEV), w.budget)
        L = s["lengths"]
    else:
        L = None
    got, st = _gpu(sv, w, L)
    t, d = _host(w.target), _host(w.draft)
    Lh = None if L is None else _host(L)
    T = _host(w.temperature)
    K = None if w.top_k is None else _host(w.top_k)
    sl = lambda x, a, b: None if x is None else x[a:b]

    def block(blk):
        a, b = blk[0], blk[-1] + 1
        return oracle.overlap_mass(t[a:b], d[a:b], sl(Lh, a, b), T[a:b], sl(K, a, b))

    res = pool_map(block, request_blocks(w.B, 8))
    ref = np.concatenate([r["overlap"] for r in res])
    st_ref = np.concatenate([r["status"] for r in res])
    _check(got, ref, st, st_ref)
    assert (st == 0).all()
    print(f"overlap {name} full size: {int(np.isfinite(got).sum())} positions of {w.B} requests compared",
          flush=True)
