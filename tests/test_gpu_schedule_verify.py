"""GPU: spec_schedule_verify (the scheduler, then verification under the budget, in one call) against
the two calls it stands for, spec_schedule_lengths then spec_verify_bounded with the same budget, on
the same stream.  Both are pinned to the oracle elsewhere; here every output must agree bit for bit
(accept_prob compared as bit patterns, so NaN marks must match too), and the lengths must also equal
the oracle's schedule.  B <= 1024 takes the path in which the scheduler writes the verify work list;
B = 1100 takes the path with the separate work-list kernel; 256 <= B <= 1024 (gamma < 64) takes the
path with no work list at all, in which each streaming workgroup derives its item from the lengths.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from oracle.scheduling import MODE_EARLY_STOP, MODE_GLOBAL
from parity import HostInputs, compare_verify, run_oracle_pooled, to_np  # noqa: F401
from workloads import make_workload

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _both(sv, w, sps, budget, mode):
    conf = w.conf.to(DEV)
    sps_d = torch.from_numpy(sps).to(DEV)
    args = (w.target, w.draft, w.draft_tokens)
    fused = sv.schedule_verify(*args, conf, sps_d, budget, mode, w.temperature, w.top_k, w.seed)
    sch = sv.schedule_lengths(conf, sps_d, budget, mode)
    two = sv.verify(*args, sch["lengths"], w.temperature, w.top_k, w.seed, max_tokens=budget)
    torch.cuda.synchronize()
    return fused, sch, two


def _check(sv, w, sps, budget, mode, with_oracle=True, verify_oracle=None):
    print(f"case B={w.B} gamma={w.gamma} V={w.V} budget={budget} mode={mode}", flush=True)
    fused, sch, two = _both(sv, w, sps, budget, mode)
    assert torch.equal(fused["lengths"], sch["lengths"])
    assert torch.equal(fused["theta"].view(torch.int64), sch["theta"].view(torch.int64))
    assert torch.equal(fused["sched_status"], sch["status"])
    for k in ("num_accepted", "out_tokens", "status"):
        assert torch.equal(fused[k], two[k]), k
    assert torch.equal(fused["accept_prob"].view(torch.int32), two["accept_prob"].view(torch.int32))
    if with_oracle:
        L_ref, _ = oracle.schedule(w.conf.cpu().numpy(), sps, budget, mode)
        assert np.array_equal(to_np(fused["lengths"]), L_ref)
        if verify_oracle is None:   # the verification outputs too (the full-size case has its own test)
            verify_oracle = w.V * w.B <= 1 << 22
        if verify_oracle:
            h = HostInputs.of_workload(w, L_ref)
            ref = run_oracle_pooled(h)
            over = _over_budget(L_ref, budget)
            for key in ("status", "accept_flags", "emit_flag", "draws"):
                ref[key] = ref[key].copy()
            ref["status"][over] = 64          # the token cap, which the oracle does not model
            ref["num_accepted"][over] = 0
            ref["out_tokens"][over] = -1
            ref["accept_prob"][over] = np.nan
            ref["accept_flags"][over] = 0
            ref["emit_flag"][over] = False
            ref["draws"][over] = 0
            compare_verify(fused, ref, inputs=h)
    return fused


def _over_budget(L, budget):
    """Requests past the token cap (index order, L + 1 tokens each): SPEC_REQ_OVER_BUDGET."""
    run = np.cumsum(L.astype(np.int64) + 1)
    return run > budget


@pytest.mark.parametrize("mode", [MODE_EARLY_STOP, MODE_GLOBAL])
def test_scheduled_small(sv, mode):
    w = make_workload("scheduled", DEV, B=96, V=5000, seed=71)
    f = _check(sv, w, w.sps, w.budget, mode)
    assert (to_np(f["status"]) == 0).all()


@pytest.mark.timeout(900)
def test_scheduled_full_size(sv):
    """The scheduled workload at its full size (B = 256, gamma = 16, V = 151936, budget 2048), in
    the very call the benchmark times: the lengths equal the oracle's schedule, and every request's
    verification outputs are compared with the oracle's directly (not only with the two-call path)."""
    w = make_workload("scheduled", DEV)
    f = _check(sv, w, w.sps, w.budget, MODE_EARLY_STOP)
    assert (to_np(f["status"]) == 0).all()
    assert int((to_np(f["lengths"]) + 1).sum()) <= w.budget
    L_ref, _ = oracle.schedule(w.conf.cpu().numpy(), w.sps, w.budget, MODE_EARLY_STOP)
    h = HostInputs.of_workload(w, L_ref)
    ref = run_oracle_pooled(h)
    s = compare_verify(f, ref, inputs=h, bound=True)
    print(f"scheduled full size: sum L = {int(L_ref.sum())}, {s}", flush=True)


def test_mixed_recipe(sv):
    # temperatures, top-k 50 and per-request seeds, with a schedule
    w = make_workload("mixed", DEV, B=300, V=3000, seed=72, with_schedule=True)
    _check(sv, w, w.sps, w.budget, MODE_GLOBAL)


@pytest.mark.timeout(600)
def test_mixed_recipe_segmented_top_k(sv):
    # rows of 129280 bf16 logits: top-k 50 rows split into four segments whose id lists are
    # merged; 300 requests take the fused emit and the request-major work list
    w = make_workload("mixed", DEV, B=300, gamma=4, V=129280, seed=79, with_schedule=True)
    _check(sv, w, w.sps, w.budget, MODE_GLOBAL, verify_oracle=True)


def test_beyond_one_workgroup(sv):
    # B > 1024: the separate work-list kernel
    w = make_workload("scheduled", DEV, B=1100, gamma=8, V=700, seed=73)
    _check(sv, w, w.sps, w.budget, MODE_EARLY_STOP)


def test_gamma_64(sv):
    # 64 draft positions (65 work-list positions) and the largest scheduler tile
    w = make_workload("scheduled", DEV, B=200, gamma=64, V=500, seed=74)
    _check(sv, w, w.sps, 4 * w.B, MODE_EARLY_STOP)


def test_budget_below_batch(sv):
    # nothing is admitted and the cap keeps only the first `budget` requests
    w = make_workload("scheduled", DEV, B=64, V=900, seed=75)
    budget = 40
    f = _check(sv, w, w.sps, budget, MODE_EARLY_STOP)
    st = to_np(f["status"])
    assert (to_np(f["lengths"]) == 0).all()
    assert (st[:budget] == 0).all() and (st[budget:] == 64).all()


def test_nothing_admitted(sv):
    # a cost table that falls faster than tau can rise: m* = 0 in both modes
    w = make_workload("scheduled", DEV, B=80, V=900, seed=76)
    b = np.arange(len(w.sps), dtype=np.float64)
    sps = np.zeros_like(b)
    sps[1:] = 1.0 / b[1:] ** 3
    for mode in (MODE_EARLY_STOP, MODE_GLOBAL):
        f = _check(sv, w, sps, w.budget, mode)
        assert (to_np(f["lengths"]) == 0).all() and (to_np(f["status"]) == 0).all()


def test_bad_confidences(sv):
    w = make_workload("scheduled", DEV, B=50, V=800, seed=77)
    w.conf[3] = float("nan")
    w.conf[7, 2] = 1.5
    # the oracle takes confidences in [0, 1] only: the two calls are the reference here
    f = _check(sv, w, w.sps, w.budget, MODE_EARLY_STOP, with_oracle=False)
    L = to_np(f["lengths"])
    assert L[3] == 0 and L[7] == 0
    assert to_np(f["sched_status"])[[3, 7]].all()


def test_fp32_logits_greedy_rows_and_top_k(sv):
    # fp32 logits; every fourth request takes the greedy rule (T = 0), every third a top-k of 7
    w = make_workload("tiny", DEV, B=64, gamma=6, V=2000, seed=78, with_schedule=True)
    assert w.target.dtype == torch.float32
    w.temperature[::4] = 0.0
    w.top_k = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    w.top_k[::3] = 7
    f = _check(sv, w, w.sps, w.budget, MODE_GLOBAL)
    assert (to_np(f["status"]) == 0).all()


@pytest.mark.parametrize("B,gamma,V,budget,mode", [
    (256, 16, 3001, None, MODE_EARLY_STOP),     # one request per streaming thread
    (700, 12, 2003, None, MODE_GLOBAL),         # two requests per thread, a ragged last chunk
    (1024, 8, 1000, None, MODE_EARLY_STOP),     # every thread's two requests
    (600, 6, 999, 450, MODE_EARLY_STOP),        # budget below the batch: the cap marks requests
    (256, 63, 500, 5000, MODE_GLOBAL),          # the most positions the derived items allow
])
def test_derived_items(sv, B, gamma, V, budget, mode):
    """Batches the fused emit serves: the streaming workgroups find their items without a work list."""
    w = make_workload("scheduled", DEV, B=B, gamma=gamma, V=V, seed=80 + B)
    b = w.budget if budget is None else budget
    f = _check(sv, w, w.sps, b, mode)
    st = to_np(f["status"])
    if b < B:
        assert (st[:b] == 0).all() and (st[b:] == 64).all()
    else:
        assert (st == 0).all()


def test_derived_items_with_greedy_rows_and_top_k(sv):
    # fp32 logits; every fourth request greedy, every third a top-k of 7; mixed temperatures
    w = make_workload("tiny", DEV, B=320, gamma=6, V=2000, seed=88, with_schedule=True)
    w.temperature[::4] = 0.0
    w.temperature[1::4] = 0.7
    w.top_k = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    w.top_k[::3] = 7
    f = _check(sv, w, w.sps, w.budget, MODE_GLOBAL)
    assert (to_np(f["status"]) == 0).all()
