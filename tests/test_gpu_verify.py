"""GPU parity of spec_verify / spec_verify_greedy / spec_philox_uniforms against the CPU oracle.

Small shapes run the oracle on every request; they span several 16-byte
vectors per thread, several emit tiles, ragged rows (odd V, so rows start off
16-byte boundaries) and every edge the method has.  The full-size workloads
compare every request with the oracle (run over a pool of host processes),
check that each flagged request took an admissible outcome, and assert the
flag bound (flagged draws under 1e-4 of draws).
"""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from parity import HostInputs, compare_verify, run_oracle, run_oracle_pooled, to_np
from workloads import make_workload

DEV = "cuda:0"
REQ_OVER_BUDGET = 64   # SPEC_REQ_OVER_BUDGET


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _run(sv, w, lengths=None):
    L = w.lengths if lengths is None else lengths
    if w.name == "greedy":
        out = sv.verify_greedy(w.target, w.draft_tokens, L)
    else:
        out = sv.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed)
    torch.cuda.synchronize()
    return out


def test_philox_bitwise(sv):
    rng = np.random.default_rng(1)
    n = 1 << 20
    seed = rng.integers(0, 2 ** 64, n, dtype=np.uint64)
    req = rng.integers(0, 2 ** 31, n).astype(np.int32)
    pos = rng.integers(0, 64, n).astype(np.int32)
    ua, ue = sv.philox_uniforms(torch.from_numpy(seed.view(np.int64)).to(DEV), torch.from_numpy(req).to(DEV),
                                torch.from_numpy(pos).to(DEV))
    ra, re = oracle.uniforms(seed, req.astype(np.uint64), pos.astype(np.uint64))
    assert (to_np(ua) == ra).all() and (to_np(ue) == re).all()


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(B=64, gamma=6, V=999, seed=5)),
    ("mid", dict(B=6, gamma=5, V=20011, seed=7)),
    ("mid", dict(B=4, gamma=3, V=60000, seed=8)),
    ("mixed", dict(B=12, gamma=4, V=30001, seed=9)),
    ("mixed", dict(B=8, gamma=3, V=129280, seed=10)),
])
def test_verify_small_all_requests(sv, name, kw):
    w = make_workload(name, DEV, **kw)
    out = _run(sv, w)
    ref = run_oracle(w)
    s = compare_verify(out, ref, inputs=HostInputs.of_workload(w))
    print(name, kw, s)


@pytest.mark.parametrize("name,kw", [
    ("greedy", dict(B=32, gamma=8, V=4099, seed=3)),
    ("greedy", dict(B=16, gamma=16, V=129280, seed=4)),
])
def test_greedy_small_all_requests(sv, name, kw):
    w = make_workload(name, DEV, **kw)
    out = _run(sv, w)
    ref = run_oracle(w)
    s = compare_verify(out, ref, check_prob=False)
    assert s["mismatches"] == 0


def test_greedy_ties_and_fp32(sv):
    rng = np.random.default_rng(2)
    B, G, V = 24, 5, 1003
    z = rng.integers(-3, 4, (B, G + 1, V)).astype(np.float32)      # many exact ties
    x = rng.integers(0, V, (B, G)).astype(np.int32)
    am = np.argmax(z, axis=-1)
    take = rng.random((B, G)) < 0.8
    x = np.where(take, am[:, :G], x).astype(np.int32)
    for dt in (torch.float32, torch.bfloat16):
        t = torch.from_numpy(z).to(DEV).to(dt)
        out = sv.verify_greedy(t, torch.from_numpy(x).to(DEV))
        torch.cuda.synchronize()
        ref = oracle.verify_greedy(t, x)
        assert (to_np(out["num_accepted"]) == ref["num_accepted"]).all()
        assert (to_np(out["out_tokens"]) == ref["out_tokens"]).all()


@pytest.mark.parametrize("rep,V,dtype", [
    (1, 777, torch.float32),      # 16 requests: the split emit; odd V, rows off 16-byte boundaries
    (16, 777, torch.float32),     # 256 requests: one fused workgroup per request
    (1, 2600, torch.bfloat16),    # bf16, V a multiple of 8: the last, partial range read as vectors
    (16, 2600, torch.bfloat16),
])
def test_verify_edge_cases(sv, rep, V, dtype):
    rng = np.random.default_rng(3)
    B, G = 16, 4
    t = rng.normal(0, 3, (B, G + 1, V)).astype(np.float32)
    d = t[:, :G] + rng.normal(0, 1, (B, G, V)).astype(np.float32)
    x = rng.integers(0, V, (B, G)).astype(np.int32)
    L = np.array([0, 1, 2, 3, 4] * 3 + [4], dtype=np.int32)
    T = np.ones(B, dtype=np.float32)
    K = np.zeros(B, dtype=np.int32)
    d[1] = t[1, :G]                        # identical distributions: everything accepted
    t[2, :, ::3] = -np.inf                 # masked tokens
    d[2, :, ::3] = -np.inf
    x[2] = 1
    T[3] = 0.05                            # very sharp
    T[4] = 7.5                             # very flat
    K[5] = 1                               # top-1
    K[6] = V                               # top-k that keeps everything
    K[7] = 3
    x[8, 0] = V                            # bad token
    T[9] = -1.0                            # bad temperature
    t[10, 0, 5] = np.nan                   # NaN in a needed row
    t[11, G, 0] = np.nan                   # NaN in a row that is not needed (L=1)
    L[11] = 1
    t[12, 0, 9] = np.inf                   # +inf
    T[13] = 0.0                            # greedy rule inside spec_verify
    L[14] = G + 1                          # bad length
    K[15] = -2                             # bad top-k
    # rep copies of the 16 cases, each copy with its own seeds
    t, d, x = np.tile(t, (rep, 1, 1)), np.tile(d, (rep, 1, 1)), np.tile(x, (rep, 1))
    L, T, K = np.tile(L, rep), np.tile(T, rep), np.tile(K, rep)
    seed = rng.integers(0, 2 ** 63, B * rep).astype(np.int64)
    tt = torch.from_numpy(t).to(DEV).to(dtype)
    dd = torch.from_numpy(d).to(DEV).to(dtype)
    args = [torch.from_numpy(a).to(DEV) for a in (x, L, T, K, seed)]
    out = sv.verify(tt, dd, *args)
    torch.cuda.synchronize()
    ref = oracle.verify(tt, dd, x, L, T, K, seed)
    compare_verify(out, ref, inputs=HostInputs.of(tt, dd, x, L, T, K, seed))
    st = to_np(out["status"]).reshape(rep, B)
    assert (st[:, 8] == oracle.STATUS_BAD_TOKEN).all() and (st[:, 9] == oracle.STATUS_BAD_TEMPERATURE).all()
    assert (st[:, 10] == oracle.STATUS_NONFINITE).all() and (st[:, 11] == 0).all()
    assert (st[:, 12] == oracle.STATUS_NONFINITE).all()
    assert (st[:, 14] == oracle.STATUS_BAD_LENGTH).all() and (st[:, 15] == oracle.STATUS_BAD_TOPK).all()
    assert (to_np(out["num_accepted"]).reshape(rep, B)[:, 1] == L[1]).all()


def test_single_token_vocabulary(sv):
    B, G, V = 3, 2, 1
    t = torch.zeros((B, G + 1, V), device=DEV)
    d = torch.zeros((B, G, V), device=DEV)
    x = torch.zeros((B, G), dtype=torch.int32, device=DEV)
    out = sv.verify(t, d, x)
    torch.cuda.synchronize()
    assert (to_np(out["num_accepted"]) == G).all()
    assert (to_np(out["out_tokens"]) == 0).all()


@pytest.mark.parametrize("V", [2, 3, 8])
def test_lossless_chi_square_on_gpu(sv, V):
    """Emitted tokens follow p_t (10^6 trials), and agree with the oracle draw for draw."""
    from scipy import stats
    rng = np.random.default_rng(200 + V)
    G, n = 2, 1_000_000
    pt = rng.dirichlet(np.ones(V) * 3, G + 1)
    pd = rng.dirichlet(np.ones(V) * 3, G)
    t = np.broadcast_to(np.log(pt).astype(np.float32), (n, G + 1, V)).copy()
    d = np.broadcast_to(np.log(pd).astype(np.float32), (n, G, V)).copy()
    x = np.stack([rng.choice(V, n, p=pd[k]) for k in range(G)], axis=1).astype(np.int32)
    out = sv.verify(torch.from_numpy(t).to(DEV), torch.from_numpy(d).to(DEV), torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    ng, tg = to_np(out["num_accepted"]), to_np(out["out_tokens"])
    pt32 = np.exp(oracle.log_probs(t[0], 1.0))
    for k in range(G + 1):
        sel = ng >= k
        obs = np.bincount(tg[sel, k], minlength=V)
        assert stats.chisquare(obs, pt32[k] * sel.sum()).pvalue > 1e-4
    ref = oracle.verify(t, d, x)
    compare_verify(out, ref, inputs=HostInputs.of(t, d, x), bound=True)


@pytest.mark.parametrize("name,kw", [
    ("mid", dict(B=4, gamma=4, V=30000, seed=21)),
    ("mixed", dict(B=12, gamma=4, V=30001, seed=9)),      # top-k rows: candidates gathered in LDS
    ("mixed", dict(B=256, gamma=3, V=129280, seed=12)),   # ... and the fused emit
])
def test_determinism(sv, name, kw):
    """The same inputs give bitwise-identical outputs, run after run."""
    w = make_workload(name, DEV, **kw)
    a = _run(sv, w)
    for _ in range(3):
        b = _run(sv, w)
        for k in a:
            assert torch.equal(a[k], b[k]) or (a[k].dtype.is_floating_point and
                                               torch.equal(torch.nan_to_num(a[k]), torch.nan_to_num(b[k]))), k


# ---- full workloads, every request ----

def _full(sv, name):
    w = make_workload(name, DEV)
    print(f"case {name}: B={w.B} gamma={w.gamma} V={w.V}", flush=True)
    out = _run(sv, w)
    h = HostInputs.of_workload(w)
    ref = run_oracle_pooled(h)
    s = compare_verify(out, ref, inputs=h, bound=True, check_prob=name != "greedy")
    print(f"{name} full size: {s}", flush=True)
    return s


@pytest.mark.timeout(900)
def test_full_mid_all_requests(sv):
    _full(sv, "mid")


@pytest.mark.timeout(900)
def test_full_greedy_all_requests(sv):
    s = _full(sv, "greedy")
    assert s["mismatches"] == 0


@pytest.mark.timeout(900)
def test_full_mixed_all_requests(sv):
    _full(sv, "mixed")


def test_draft_token_outside_the_draft_top_k(sv):
    """The edge rules of the ratio (DSpark paper, §2.1, with top-k): a draft token outside the
    draft's kept set but inside the target's has p_d(x) = 0 < p_t(x), so r = 1 and it is always
    accepted; one inside the draft's kept set but outside the target's has r = 0 and is always
    rejected."""
    rng = np.random.default_rng(44)
    B, G, V, K = 64, 4, 5000, 5
    t = rng.normal(0, 3, (B, G + 1, V)).astype(np.float32)
    d = t[:, :G] + rng.normal(0, 0.5, (B, G, V)).astype(np.float32)
    x = np.zeros((B, G), dtype=np.int32)
    want = np.zeros((B, G))
    for i in range(B):
        for k in range(G):
            top_t = np.argsort(-t[i, k], kind="stable")[:K]
            if (i + k) % 2 == 0:
                v = int(top_t[1])
                d[i, k, v] = -20.0          # out of the draft's top-k, still in the target's
                want[i, k] = 1.0
            else:
                v = int(np.argsort(-d[i, k], kind="stable")[0])
                t[i, k, v] = -20.0          # in the draft's top-k, out of the target's
                want[i, k] = 0.0
            x[i, k] = v
    Kv = np.full(B, K, dtype=np.int32)
    T = rng.uniform(0.6, 1.2, B).astype(np.float32)
    seed = rng.integers(0, 2 ** 63, B).astype(np.int64)
    for dt in (torch.float32, torch.bfloat16):
        tt = torch.from_numpy(t).to(DEV).to(dt)
        dd = torch.from_numpy(d).to(DEV).to(dt)
        args = [torch.from_numpy(a).to(DEV) for a in (x, np.full(B, G, np.int32), T, Kv, seed)]
        out = sv.verify(tt, dd, *args)
        torch.cuda.synchronize()
        ref = oracle.verify(tt, dd, x, None, T, Kv, seed)
        compare_verify(out, ref, inputs=HostInputs.of(tt, dd, x, None, T, Kv, seed))
        r = to_np(out["accept_prob"])
        assert (ref["accept_prob"] == want).all()
        assert (r == want).all()
        n = to_np(out["num_accepted"])
        first = np.where((want == 0).any(axis=1), np.argmax(want == 0, axis=1), G)
        assert (n == first).all()


def test_nearly_identical_rows_take_the_exact_residual_path(sv):
    """Draft equal to the target except one low-probability token: almost every
    token's residual sign sits inside the classification margin, so the emit
    must fall back to weighing every token exactly."""
    rng = np.random.default_rng(41)
    B, G, V = 256, 1, 40000
    base = rng.normal(0, 3, (1, G + 1, V)).astype(np.float32)
    t = np.repeat(base, B, axis=0)
    d = t[:, :G].copy()
    x = np.zeros((B, G), dtype=np.int32)
    lo = int(np.argmin(base[0, 0]))
    d[:, 0, lo] += 12.0                 # the draft over-weights one token
    x[:, 0] = lo                        # ... and proposes it: r = p_t/p_d is small
    for dt in (torch.float32, torch.bfloat16):
        tt = torch.from_numpy(t).to(DEV).to(dt)
        dd = torch.from_numpy(d).to(DEV).to(dt)
        out = sv.verify(tt, dd, torch.from_numpy(x).to(DEV))
        torch.cuda.synchronize()
        ref = oracle.verify(tt, dd, x)
        s = compare_verify(out, ref)
        assert (ref["num_accepted"] == 0).sum() > B // 2, s   # mostly rejected -> residual draws



def _segmented_topk_case(rng, B, G, V):
    """Sampling requests with top-k, on rows long enough to be split into segments (top_k <= 64
    merges per-segment id lists; larger top_k streams rows whole), with the rows that take the
    fall-backs: candidate and id-list overflow, ties at the cut, the kept set inside one segment,
    invalid values in a later segment, greedy requests with a top-k."""
    t = rng.normal(0, 3, (B, G + 1, V)).astype(np.float32)
    d = t[:, :G] + rng.normal(0, 0.8, (B, G, V)).astype(np.float32)
    Ks = [1, 2, 17, 50, 64, 65, 200, 0, V - 1, V]
    K = np.array([Ks[i % len(Ks)] for i in range(B)], dtype=np.int32)
    T = rng.uniform(0.6, 1.2, B).astype(np.float32)
    L = rng.integers(0, G + 1, B).astype(np.int32)
    q = V // 4
    for base in range(0, B, 16):
        if base + 15 >= B:
            break
        r = base
        T[r], K[r] = 0.0, 50                                        # greedy rule: top-k ignored
        r += 1
        t[r] = rng.integers(-3, 4, t[r].shape)                      # massive ties: candidate overflow
        d[r] = rng.integers(-3, 4, d[r].shape)
        K[r] = 50
        r += 1
        t[r, :, 2 * q:2 * q + 100] = t[r].max() + 5.0                # 100 tokens tie at the cut: id overflow
        K[r] = 50
        r += 1
        t[r, :, V - 200:] += 10.0                                    # every kept token in the last segment
        d[r, :, V - 200:] += 10.0
        K[r] = 40
        r += 1
        t[r, 0, 3 * q + 7] = np.nan                                  # NaN in a later segment
        K[r], L[r] = 50, G
        r += 1
        d[r, 0, q + 3] = np.inf                                      # +inf in a draft row's second segment
        K[r], L[r] = 50, G
        r += 1
        K[r], L[r] = 1, 0                                            # top-1, appended token only
        r += 1
        d[r] = t[r, :G]                                              # identical rows: all accepted
        K[r], L[r] = 64, G
        r += 1
        K[r] = 64                                                    # 11 values tie at the 60th largest,
        for k in range(G + 1):                                       # spread over the segments
            v60 = np.sort(t[r, k])[::-1][59]
            t[r, k, rng.choice(V, 10, replace=False)] = v60
        r += 1
        t[r, :, ::97] = -np.inf                                      # -inf logits (valid) in every segment,
        d[r, :, ::89] = -np.inf                                      # whole 16-byte vectors of them too
        t[r, :, q:q + 64] = -np.inf
        d[r, :, 3 * q:3 * q + 64] = -np.inf
        K[r], L[r] = 50, G
        r += 1
        T[r], L[r] = 0.0, G                                          # greedy rows: NaN in a later segment,
        t[r, 0, 2 * q + 11] = np.nan
        r += 1
        T[r], L[r] = 0.0, G                                          # +inf in target row 1's last segment,
        t[r, 1, 3 * q + 5] = np.inf
        r += 1
        T[r], L[r] = 0.0, G                                          # -inf logits, valid
        t[r, :, ::5] = -np.inf
        t[r, :, 2 * q:2 * q + 64] = -np.inf
    x = np.zeros((B, G), dtype=np.int32)
    for i in range(B):
        for k in range(G):
            if K[i] > 0 and rng.random() < 0.7:     # mostly inside the draft's kept set
                x[i, k] = int(np.argsort(-d[i, k], kind="stable")[rng.integers(0, min(int(K[i]), 5))])
            else:
                x[i, k] = int(rng.integers(0, V))
    for base in range(0, B - 15, 16):
        x[base + 7] = np.argmax(d[base + 7], axis=-1)              # in the kept set of both rows
    seed = rng.integers(0, 2 ** 63, B).astype(np.int64)
    return t, d, x, L, T, K, seed


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,V,dtype", [
    (32, 129280, torch.bfloat16),    # four segments per row; split emit
    (256, 129280, torch.bfloat16),   # fused emit
    (32, 65536, torch.float32),      # fp32 rows, four segments
    (48, 30001, torch.float32),      # fp32, two segments, rows off 16-byte boundaries
])
def test_segmented_topk_all_requests(sv, B, V, dtype):
    rng = np.random.default_rng(B + V)
    G = 4 if B <= 48 else 2
    t, d, x, L, T, K, seed = _segmented_topk_case(rng, B, G, V)
    tt = torch.from_numpy(t).to(DEV).to(dtype)
    dd = torch.from_numpy(d).to(DEV).to(dtype)
    args = [torch.from_numpy(a).to(DEV) for a in (x, L, T, K, seed)]
    out = sv.verify(tt, dd, *args)
    torch.cuda.synchronize()
    h = HostInputs.of(tt, dd, x, L, T, K, seed)
    ref = run_oracle_pooled(h)
    s = compare_verify(out, ref, inputs=h)
    print(B, V, dtype, s, flush=True)
    st = to_np(out["status"])
    for base in range(0, B - 15, 16):
        assert st[base + 4] == oracle.STATUS_NONFINITE and st[base + 5] == oracle.STATUS_NONFINITE
        assert int(to_np(out["num_accepted"])[base + 7]) == G
        assert st[base + 9] == 0 and st[base + 12] == 0                      # -inf is a valid logit
        assert st[base + 10] == oracle.STATUS_NONFINITE and st[base + 11] == oracle.STATUS_NONFINITE


def _flatten(w, L):
    Lh = to_np(L).astype(np.int64)
    G = w.gamma
    ok = (Lh >= 0) & (Lh <= G)
    trows = torch.cat([w.target[i, :Lh[i] + 1] for i in range(w.B) if ok[i]], 0)
    drows = [w.draft[i, :Lh[i]] for i in range(w.B) if ok[i] and Lh[i] > 0]
    drows = torch.cat(drows, 0) if drows else w.draft[:0, 0]
    return trows.contiguous(), drows.contiguous()


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(B=40, gamma=6, V=999, seed=5)),
    ("mid", dict(B=6, gamma=5, V=20011, seed=7)),
    ("mixed", dict(B=12, gamma=4, V=30001, seed=9)),
    ("mixed", dict(B=8, gamma=3, V=129280, seed=12)),     # segmented top-k rows
    ("scheduled", dict(B=300, gamma=8, V=4096, seed=11)),
])
def test_flat_layout_equals_padded(sv, name, kw):
    """spec_verify_flat on the rows gathered request after request gives spec_verify's outputs
    (and the oracle's); a bad length counts as no rows.  Bit for bit when rows are a multiple of
    16 bytes; otherwise the two layouts start rows at other 16-byte offsets, which changes the
    order of the row sums, so r agrees to rounding and the decisions are held to the oracle."""
    w = make_workload(name, DEV, **kw)
    rng = np.random.default_rng(91)
    Lh = rng.integers(0, w.gamma + 1, w.B).astype(np.int32)
    Lh[rng.random(w.B) < 0.05] = w.gamma + 2
    L = torch.from_numpy(Lh).to(DEV)
    ref = sv.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed)
    trows, drows = _flatten(w, L)
    got = sv.verify_flat(trows, drows, w.draft_tokens, L, w.temperature, w.top_k, w.seed)
    torch.cuda.synchronize()
    a, b = to_np(got["accept_prob"]), to_np(ref["accept_prob"])
    if (w.V * w.elem_bytes) % 16 == 0:
        for k in ("num_accepted", "out_tokens", "status"):
            assert (to_np(got[k]) == to_np(ref[k])).all(), k
        assert ((a == b) | (np.isnan(a) & np.isnan(b))).all()
    else:
        assert (to_np(got["status"]) == to_np(ref["status"])).all()
        assert (np.isnan(a) == np.isnan(b)).all()
        ok = ~np.isnan(a)
        assert (np.abs(a[ok] - b[ok]) <= 1e-6 * np.abs(b[ok]) + 1e-12).all()
    o = run_oracle(w, lengths=L)
    compare_verify(got, o)


@pytest.mark.parametrize("name,kw,bounds", [
    ("scheduled", dict(B=300, gamma=8, V=4096, seed=11), (1, 37, 299, 10 ** 6)),
    ("mid", dict(B=6, gamma=5, V=20011, seed=7), (1, 5, 36)),
    ("mixed", dict(B=12, gamma=4, V=30001, seed=9), (3, 60)),
    ("mixed", dict(B=8, gamma=3, V=129280, seed=12), (2, 17)),   # segmented top-k rows
])
def test_token_cap(sv, name, kw, bounds):
    """spec_verify_bounded: requests in index order add L_i + 1 (valid lengths only) to a running
    sum; from the first that passes the cap on, requests with a valid length get OVER_BUDGET and
    failed-request outputs.  Every request that fits must equal spec_verify's outputs bit for bit
    (the cap also sizes the streaming grid, so both a tight and a loose cap are tried)."""
    w = make_workload(name, DEV, **kw)
    rng = np.random.default_rng(5)
    Lh = rng.integers(0, w.gamma + 1, w.B).astype(np.int32)
    Lh[rng.random(w.B) < 0.05] = w.gamma + 2            # bad lengths count as no rows
    L = torch.from_numpy(Lh).to(DEV)
    ref = sv.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed)
    torch.cuda.synchronize()
    valid = (Lh >= 0) & (Lh <= w.gamma)
    run = np.cumsum(np.where(valid, Lh.astype(np.int64) + 1, 0))
    for b in bounds:
        got = sv.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed, max_tokens=b)
        torch.cuda.synchronize()
        over = valid & (run > b)
        assert not over.any() or np.all(over[np.argmax(over):] == valid[np.argmax(over):])   # a suffix
        keep = torch.from_numpy(~over).to(DEV)
        for k in ("num_accepted", "out_tokens", "status"):
            assert torch.equal(got[k][keep], ref[k][keep]), (b, k)
        a_got = torch.nan_to_num(got["accept_prob"], nan=-1.0)
        assert torch.equal(a_got[keep], torch.nan_to_num(ref["accept_prob"], nan=-1.0)[keep]), b
        o = torch.from_numpy(over).to(DEV)
        assert (got["status"][o] == REQ_OVER_BUDGET).all() and (got["num_accepted"][o] == 0).all()
        assert (got["out_tokens"][o] == -1).all() and torch.isnan(got["accept_prob"][o]).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype,V,G", [
    (torch.bfloat16, 524288, 64),    # the largest bf16 rows and the longest block the library takes
    (torch.float32, 262144, 8),      # the largest fp32 rows
])
def test_maximum_vocabulary_and_block(sv, dtype, V, G):
    """Every position verified on rows of the largest vocabulary: a sampling request, a top-k of 64
    (segmented rows, which at this size take the counting fall-back of the merge) and the greedy
    rule, against the oracle."""
    rng = np.random.default_rng(V + G)
    B = 3
    t = rng.standard_normal((B, G + 1, V), dtype=np.float32) * np.float32(3.0)
    d = t[:, :G] + rng.standard_normal((B, G, V), dtype=np.float32) * np.float32(0.5)
    T = np.array([1.0, 0.8, 0.0], dtype=np.float32)
    K = np.array([0, 64, 0], dtype=np.int32)
    L = np.full(B, G, dtype=np.int32)
    x = np.argmax(d, axis=-1).astype(np.int32)            # the draft's top token: mostly accepted
    x[:, 1::3] = rng.integers(0, V, (B, len(range(1, G, 3))))   # a random token: mostly rejected
    seed = rng.integers(0, 2 ** 63, B).astype(np.int64)
    tt = torch.from_numpy(t).to(DEV).to(dtype)
    dd = torch.from_numpy(d).to(DEV).to(dtype)
    del t, d
    args = [torch.from_numpy(a).to(DEV) for a in (x, L, T, K, seed)]
    out = sv.verify(tt, dd, *args)
    torch.cuda.synchronize()
    h = HostInputs.of(tt, dd, x, L, T, K, seed)
    ref = run_oracle_pooled(h, block=1)
    s = compare_verify(out, ref, inputs=h)
    print(dtype, V, G, s, flush=True)
    assert (to_np(out["status"]) == 0).all()


# ---- a closed form at the workloads' vocabulary size ----

def _closed_form_case(B, G, V, seed):
    """Target rows uniform (logits 0); draft row k of request i uniform on a set S of |S| tokens
    (logit 0 there, -inf elsewhere), |S| cycling through V/100, V/2 and V-1; draft tokens from S.
    Then r_k = |S|/V exactly, and the emitted token has a closed form: after a rejection at n the
    residual max(0, 1/V - 1/|S|) is 1/V on the complement of S, so the token is the complement token
    of rank floor(u_emit * (V - |S|)); after full acceptance it is floor(u_emit * V)."""
    rng = np.random.default_rng(seed)
    sizes = np.array([V // 100, V // 2, V - 1])
    target = torch.zeros((B, G + 1, V), dtype=torch.bfloat16)
    draft = torch.full((B, G, V), float("-inf"), dtype=torch.bfloat16)
    tokens = np.empty((B, G), dtype=np.int64)
    sets = {}
    for i in range(B):
        s = int(sizes[i % 3])
        for k in range(G):
            S = np.sort(rng.choice(V, size=s, replace=False))
            sets[i, k] = S
            draft[i, k, torch.from_numpy(S)] = 0.0
            tokens[i, k] = S[rng.integers(s)]
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    return target, draft, tokens, sets, seeds, sizes


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [256, 40])   # the fused emit, and the split emit of smaller batches
def test_residual_closed_form_at_large_vocabulary(sv, B):
    G, V = 3, 151936
    target, draft, tokens, sets, seeds, sizes = _closed_form_case(B, G, V, 900 + B)
    print(f"case closed form B={B} G={G} V={V}", flush=True)
    out = sv.verify(target.to(DEV), draft.to(DEV), torch.from_numpy(tokens.astype(np.int32)).to(DEV), None,
                    torch.ones(B, device=DEV), None, torch.from_numpy(seeds).to(DEV))
    torch.cuda.synchronize()
    n_g, t_g, r_g, st = (to_np(out[k]) for k in ("num_accepted", "out_tokens", "accept_prob", "status"))
    assert (st == 0).all()
    flagged = checked = 0
    kinds = set()
    for i in range(B):
        s = int(sizes[i % 3])
        r = s / V
        np.testing.assert_allclose(r_g[i], r, rtol=1e-5)
        u_acc, u_emit = oracle.uniforms(np.full(G + 1, seeds[i], dtype=np.int64).view(np.uint64),
                                        np.full(G + 1, i), np.arange(G + 1))
        if (np.abs(u_acc[:G] - r) < oracle.FLAG_ACCEPT_WINDOW).any():
            flagged += 1
            continue
        n = next((k for k in range(G) if not u_acc[k] < r), G)
        assert n_g[i] == n, (i, n_g[i], n)
        if n < G:
            m = V - s
            pos = u_emit[n] * m
            want = int(np.setdiff1d(np.arange(V), sets[i, n])[int(np.floor(pos))])
        else:
            m = V
            pos = u_emit[G] * V
            want = int(np.floor(pos))
        if abs(pos - round(pos)) < oracle.FLAG_EMIT_WINDOW * m:
            flagged += 1
            continue
        assert t_g[i, n] == want, (i, n, t_g[i, n], want)
        assert (t_g[i, :n] == tokens[i, :n]).all() and (t_g[i, n + 1:] == -1).all()
        checked += 1
        kinds.add((s, n < G))
    print(f"closed form B={B}: {checked} requests checked, {flagged} flagged, outcomes {sorted(kinds)}", flush=True)
    assert flagged <= 1 and checked >= B - 1
    assert any(rej for _, rej in kinds) and any(not rej for _, rej in kinds)
