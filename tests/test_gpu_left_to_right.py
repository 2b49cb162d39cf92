"""GPU: spec_schedule_verify with SPEC_VERIFY_LEFT_TO_RIGHT -- the walk that stops at the first
rejection (DSpark paper §2.1), streamed in two passes (positions 0 .. c-1 of every request, then the
rest of the requests whose walk goes on; c = 3, or 2 for rows of more than 8 segments) -- against oracle.verify_left_to_right on the same inputs
and the lengths of the oracle's schedule: accepted lengths and tokens bit for bit except flagged
draws (each checked to be an admissible outcome), accept_prob within 1e-5 up to the first
rejection and NaN after it, status words equal.  Bad rows are planted after, at and before the
first rejection, in rows of both passes.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from oracle.scheduling import MODE_EARLY_STOP, MODE_GLOBAL
from parity import HostInputs, compare_verify, run_oracle_pooled, to_np
from workloads import make_workload

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _run(sv, w, mode=MODE_EARLY_STOP, left_to_right=True):
    conf = w.conf.to(DEV)
    sps = torch.from_numpy(w.sps).to(DEV)
    out = sv.schedule_verify(w.target, w.draft, w.draft_tokens, conf, sps, w.budget, mode, w.temperature,
                             w.top_k, w.seed, left_to_right=left_to_right)
    torch.cuda.synchronize()
    return out


def _check(sv, w, mode=MODE_EARLY_STOP, bound=False):
    print(f"case B={w.B} gamma={w.gamma} V={w.V} budget={w.budget} mode={mode}", flush=True)
    out = _run(sv, w, mode)
    L_ref, _ = oracle.schedule(w.conf.cpu().numpy(), w.sps, w.budget, mode)
    assert np.array_equal(to_np(out["lengths"]), L_ref)
    h = HostInputs.of_workload(w, L_ref)
    ref = run_oracle_pooled(h, left_to_right=True)
    s = compare_verify(out, ref, inputs=h, bound=bound, left_to_right=True)
    # the walk's accepted lengths and tokens are the full verification's
    full = _run(sv, w, mode, left_to_right=False)
    same = (to_np(full["num_accepted"]) == to_np(out["num_accepted"])) & \
        (to_np(full["out_tokens"]) == to_np(out["out_tokens"])).all(axis=1)
    flagged = ref["emit_flag"] | (ref["accept_flags"] > 0)
    valid = to_np(full["status"]) == 0   # bad rows anywhere fail the full verification
    assert (same | flagged | ~valid).all()
    n = to_np(out["num_accepted"])
    rf, rl = to_np(full["accept_prob"]), to_np(out["accept_prob"])
    for i in np.nonzero(same & valid)[0]:
        upto = min(int(n[i]) + 1, int(L_ref[i]))
        assert np.array_equal(rf[i, :upto].view(np.int32), rl[i, :upto].view(np.int32))
        assert np.isnan(rl[i, upto:]).all()
    return out, ref, h, s


@pytest.mark.timeout(900)
def test_full_size_every_request(sv):
    """The scheduled workload at full size (B = 256, gamma = 16, V = 151936 bf16, budget 2048)."""
    w = make_workload("scheduled", DEV)
    out, ref, h, s = _check(sv, w, bound=True)
    assert (to_np(out["status"]) == 0).all()
    L = h.lengths
    n = ref["num_accepted"]
    print(f"left-to-right full size: sum L = {int(L.sum())}, rejected before position 3: "
          f"{int(((n < 3) & (n < L)).sum())}, {s}", flush=True)


@pytest.mark.parametrize("B,gamma,V,mode,seed", [
    (256, 16, 3001, MODE_EARLY_STOP, 301),   # one request per streaming thread, ragged rows
    (300, 8, 4096, MODE_GLOBAL, 302),
    (700, 12, 2003, MODE_GLOBAL, 303),       # two requests per thread
    (1024, 8, 1000, MODE_EARLY_STOP, 304),   # every thread's two requests
    (256, 63, 500, MODE_GLOBAL, 305),        # the most positions the derived items allow
    (256, 3, 999, MODE_GLOBAL, 308),         # the first pass holds every draft position
    (256, 2, 999, MODE_GLOBAL, 306),         # a first pass of two positions
    (256, 1, 999, MODE_GLOBAL, 307),         # one draft position: a first pass of one position
    (256, 4, 262144, MODE_EARLY_STOP, 309),  # rows of 10 segments: a first pass of two positions
])
def test_shapes(sv, B, gamma, V, mode, seed):
    w = make_workload("scheduled", DEV, B=B, gamma=gamma, V=V, seed=seed)
    if gamma == 63:
        w.budget = 5000
    out, ref, h, s = _check(sv, w, mode)
    assert (to_np(out["status"]) == 0).all()
    L = h.lengths
    assert (L >= min(3, gamma)).any()   # some walks reach the second pass


def test_fp32_greedy_rows_and_temperatures(sv):
    # fp32 logits; every fourth request takes the greedy rule, temperatures mixed
    w = make_workload("tiny", DEV, B=320, gamma=6, V=2000, seed=311, with_schedule=True)
    w.temperature[::4] = 0.0
    w.temperature[1::4] = 0.7
    w.top_k = None
    out, ref, h, s = _check(sv, w, MODE_GLOBAL)
    assert (to_np(out["status"]) == 0).all()


def test_bad_rows_after_at_and_before_the_first_rejection(sv):
    """NaN / +inf rows planted where the walk does and does not reach, in rows of both passes."""
    w = make_workload("scheduled", DEV, B=256, gamma=12, V=3000, seed=321)
    L_ref, _ = oracle.schedule(w.conf.cpu().numpy(), w.sps, w.budget, MODE_EARLY_STOP)
    clean = run_oracle_pooled(HostInputs.of_workload(w, L_ref), left_to_right=True)
    n = clean["num_accepted"]
    L = L_ref.astype(np.int64)
    plans = []   # (request, row kind, position, value, walk reaches it)
    picks = {
        "after_rej_first_pass": np.nonzero((n == 0) & (L >= 2))[0],      # row 1 streamed, never reached
        "after_rej_second_pass": np.nonzero((n >= 3) & (n + 1 < L))[0],  # rows past a later rejection
        "at_rej_second_pass": np.nonzero((n >= 3) & (n < L))[0],
        "before_rej": np.nonzero((n >= 1) & (n < L))[0],
        "bonus_row": np.nonzero((n == L) & (L >= 1))[0],
        "bonus_row_first_pass": np.nonzero((n == L) & (L == 1))[0],
    }
    used = set()

    def take(key):
        for i in picks[key]:
            if int(i) not in used:
                used.add(int(i))
                return int(i)
        return None

    i = take("after_rej_first_pass")
    if i is not None:
        plans += [(i, "target", 1, np.nan, False), (i, "draft", 1, np.inf, False)]
    i = take("after_rej_second_pass")
    if i is not None:
        plans += [(i, "target", int(n[i]) + 1, np.nan, False), (i, "draft", int(n[i]) + 1, np.nan, False)]
    i = take("at_rej_second_pass")
    if i is not None:
        plans += [(i, "draft", int(n[i]), np.nan, True)]
    i = take("before_rej")
    if i is not None:
        plans += [(i, "target", int(n[i]) - 1, np.inf, True)]
    i = take("bonus_row")
    if i is not None:
        plans += [(i, "target", int(L[i]), np.nan, True)]
    i = take("bonus_row_first_pass")
    if i is not None:
        plans += [(i, "target", 1, np.nan, True)]
    assert len({p[0] for p in plans}) >= 5, picks
    for i, kind, k, val, _ in plans:
        rows = w.target if kind == "target" else w.draft
        rows[i, k, 17] = val
    out, ref, h, s = _check(sv, w)
    st = to_np(out["status"])
    for i, kind, k, val, reached in plans:
        want = oracle.STATUS_NONFINITE if reached else 0
        assert st[i] == want, (i, kind, k, val, reached, st[i])
    others = np.setdiff1d(np.arange(w.B), [p[0] for p in plans])
    assert (st[others] == 0).all()
    # the full verification reports every planted row
    full = _run(sv, w, left_to_right=False)
    assert (to_np(full["status"])[[p[0] for p in plans]] == oracle.STATUS_NONFINITE).all()


def test_repeat_calls_are_bitwise_identical(sv):
    w = make_workload("scheduled", DEV, B=512, gamma=10, V=5000, seed=331)
    a = _run(sv, w)
    b = _run(sv, w)
    for k in ("lengths", "num_accepted", "out_tokens", "status"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["accept_prob"].view(torch.int32), b["accept_prob"].view(torch.int32))


def test_nothing_admitted_every_walk_is_the_fresh_token(sv):
    """A cost table that falls faster than tau can rise: every length is 0, the first pass streams
    target row 0 alone, no walk goes on (the second pass has no items) and every request draws its
    fresh token from target row 0."""
    w = make_workload("scheduled", DEV, B=300, gamma=8, V=2500, seed=341)
    b = np.arange(len(w.sps), dtype=np.float64)
    sps = np.zeros_like(b)
    sps[1:] = 1.0 / b[1:] ** 3
    w.sps = sps
    out, ref, h, s = _check(sv, w, MODE_EARLY_STOP)
    assert (to_np(out["lengths"]) == 0).all() and (to_np(out["status"]) == 0).all()
    assert (to_np(out["num_accepted"]) == 0).all() and np.isnan(to_np(out["accept_prob"])).all()


def test_bad_rows_with_every_thread_holding_two_requests(sv):
    """B = 1024 (each streaming workgroup's thread covers two requests' first-item words): NaN rows
    planted in a quarter of the requests, at positions before, at and after their first rejection."""
    w = make_workload("scheduled", DEV, B=1024, gamma=8, V=1500, seed=351)
    L_ref, _ = oracle.schedule(w.conf.cpu().numpy(), w.sps, w.budget, MODE_EARLY_STOP)
    clean = run_oracle_pooled(HostInputs.of_workload(w, L_ref), left_to_right=True)
    n = clean["num_accepted"]
    rng = np.random.default_rng(5)
    planted = []
    for i in rng.choice(w.B, size=256, replace=False):
        i = int(i)
        L = int(L_ref[i])
        k = int(rng.integers(0, L + 1))
        kind = "draft" if (k < L and rng.random() < 0.5) else "target"
        (w.target if kind == "target" else w.draft)[i, k, int(rng.integers(w.V))] = float("nan")
        planted.append((i, kind, k, k <= int(n[i])))
    out, ref, h, s = _check(sv, w, MODE_EARLY_STOP)
    st = to_np(out["status"])
    for i, kind, k, reached in planted:
        assert st[i] == (oracle.STATUS_NONFINITE if reached else 0), (i, kind, k, reached)
    assert any(r for *_, r in planted) and any(not r for *_, r in planted)


def test_top_k_is_refused(sv):
    w = make_workload("scheduled", DEV, B=256, gamma=4, V=1000, seed=361)
    w.top_k = torch.full((w.B,), 7, dtype=torch.int32, device=DEV)
    with pytest.raises(sv.SpecError):
        _run(sv, w)
