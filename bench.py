"""Benchmark: one step = the whole hot path on the confidence-scheduled workload.

Workload (B=256 requests, gamma=16, V=151936, bf16 logits, 2048-token verify
budget): one spec_schedule_verify call, in which the scheduler picks per-request
verify lengths from the confidences and the engine cost table (its last kernel
also writing the verify work list), then the verifier verifies exactly the
selected prefixes (row statistics, acceptance tests, first rejection,
correction / appended token).  --two-calls makes the same step from
spec_schedule_lengths and spec_verify_bounded.  Inputs are resident in HBM
before timing.

Prints ONE JSON line:
  value      verified draft positions per second (sum of scheduled lengths / step time)
  roofline   achieved HBM GB/s of the row-streaming kernel (algorithmic bytes of the
             rows it reads, each once, / its average launch time from HIP events
             recorded around it on the launch stream), against 8 TB/s
             and against the rate a plain read kernel reaches on the same bytes here
  cpu_baseline  the CPU oracle (numpy fp64) on the same workload, in verified draft
             positions per second: over a pool of worker processes (one per core
             used) and single-threaded on a bounded sample

Two copies of the logits are used alternately so consecutive steps never read
rows still resident in the 256 MB last-level cache.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps first: the GPU's clocks reach their steady state within ~50 steps")
    p.add_argument("--config", default="scheduled")
    p.add_argument("--copies", type=int, default=2)
    p.add_argument("--event-every", type=int, default=8,
                   help="time the streaming dispatch with HIP events on every N-th timed step (events on a "
                        "dispatch hold the stream for a few microseconds before and after it)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-overlap", action="store_true", help="skip the overlap-mass measurement")
    p.add_argument("--no-draft", action="store_true", help="skip the draft-sampler measurement")
    p.add_argument("--no-sts", action="store_true", help="skip the temperature-scaling measurement")
    p.add_argument("--two-calls", action="store_true",
                   help="scheduler and verification as two calls instead of spec_schedule_verify")
    p.add_argument("--left-to-right", action="store_true",
                   help="time the step as spec_schedule_verify with SPEC_VERIFY_LEFT_TO_RIGHT: the walk that stops "
                        "at the first rejection, streamed in two passes (rows after the first rejection not read)")
    p.add_argument("--no-ltr", action="store_true", help="skip the left-to-right side measurement")
    p.add_argument("--pool", type=int, default=0,
                   help="worker processes for the pooled CPU-oracle timing (0: the host cores this process "
                        "may use, at most 16, the CPU share of a one-GPU box)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (for HBM counter scaling)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "stream_kernel_traffic.json"))
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark measures one GPU (the verification kernels need no "
                                   "collective; a batch shards by request); run with --gpus 1"}))
        sys.exit(2)

    import torch
    import draft_verification_04_amd as sv
    import oracle
    from workloads import make_workload

    dev = torch.device("cuda:0")
    sv.load_library()
    torch.cuda.synchronize()
    w = make_workload(args.config, dev)
    greedy = w.draft is None  # the greedy workload has no draft logits: spec_verify_greedy
    copies = [(w.target, w.draft)]
    for c in range(1, args.copies):
        copies.append((w.target.clone(), None if greedy else w.draft.clone()))
    sps = torch.from_numpy(w.sps).to(dev) if w.sps is not None else None
    B, G, V = w.B, w.gamma, w.V
    es = w.elem_bytes
    ws = torch.empty(max(sv.verify_workspace_bytes(B, G, V),
                         int(sv.load_library().spec_verify_greedy_workspace_size(B, G))), dtype=torch.uint8, device=dev)
    sch_ws = torch.empty(max(256, sv.load_library().spec_schedule_workspace_size(B, G)), dtype=torch.uint8,
                         device=dev)
    sch_out = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ver_out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, G + 1), dtype=torch.int32, device=dev),
                   accept_prob=torch.empty((B, G), dtype=torch.float32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    stream = torch.cuda.current_stream()

    fused_out = dict(ver_out, lengths=sch_out["lengths"], theta=sch_out["theta"], sched_status=sch_out["status"])

    def step(idx, events=None):
        tgt, drf = copies[idx % len(copies)]
        if w.conf is not None and not greedy and not args.two_calls:
            # scheduler, then verification under its token budget, in one call
            sv.schedule_verify(tgt, drf, w.draft_tokens, w.conf, sps, w.budget, sv.SPEC_SCHED_EARLY_STOP,
                               w.temperature, w.top_k, w.seed, out=fused_out, workspace=ws,
                               sched_workspace=sch_ws, stream=stream, events=events,
                               left_to_right=args.left_to_right)
            return
        if w.conf is not None:
            sv.schedule_lengths(w.conf, sps, w.budget, out=sch_out, stream=stream, workspace=sch_ws)
            L = sch_out["lengths"]
        else:
            L = None
        if greedy:
            sv.verify_greedy(tgt, w.draft_tokens, L, out=ver_out, workspace=ws, stream=stream)
        else:
            # lengths from the scheduler: its token budget bounds sum (L_i + 1)
            sv.verify(tgt, drf, w.draft_tokens, L, w.temperature, w.top_k, w.seed, out=ver_out, workspace=ws,
                      stream=stream, events=events, max_tokens=w.budget if w.conf is not None else None)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    K = args.steps
    from draft_verification_04_amd.hipevents import HipEvent
    every = max(1, args.event_every)
    evs = [(HipEvent(), HipEvent()) if s % every == 0 else None for s in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(K):
        step(s, evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / K
    if greedy:  # no events inside the greedy call: the whole call bounds the streaming kernel
        ms_stream = ms_stream_median = ms_step
    else:
        per_launch = [e[0].elapsed_ms(e[1]) for e in evs if e is not None]
        ms_stream = float(np.mean(per_launch))
        ms_stream_median = float(np.median(per_launch))

    L = sch_out["lengths"].cpu().numpy().astype(np.int64) if w.conf is not None else np.full(B, G)
    positions = int(L.sum())
    rows = int((L + 1).sum()) if greedy else int((2 * L + 1).sum())
    rows_scheduled = rows
    ltr = args.left_to_right and w.conf is not None and not greedy and not args.two_calls
    if ltr:
        rows = ltr_rows(L, ver_out["num_accepted"].cpu().numpy(), G, ltr_first_pass(G, V, es))
    alg_bytes = rows * V * es
    achieved = alg_bytes / (ms_stream * 1e-3) / 1e9
    # the whole step (scheduler, streaming, acceptance, emit and every kernel boundary) against the
    # same algorithmic bytes: the fused verify path's rate
    path_gbps = alg_bytes / (ms_step * 1e-3) / 1e9
    value = positions / (ms_step * 1e-3)

    # the walk's step right after the headline's, under the same conditions
    walk = None
    if not args.no_ltr and not ltr and w.conf is not None and not greedy and w.top_k is None \
            and 256 <= B <= 1024 and G < 64:
        walk = ltr_leg(sv, torch, w, copies, sps, ws, sch_ws, stream, ms_step, L)
    ceiling = read_ceiling(sv, torch, copies, alg_bytes, stream)
    overlap = None
    if not args.no_overlap and not greedy:
        overlap = overlap_leg(sv, torch, w, copies, sch_out["lengths"] if w.conf is not None else None, stream)
    async_sched = async_scheduler_leg(sv, torch, w, sps, stream) if w.conf is not None else None
    draft = None
    if not args.no_draft:
        draft = draft_leg(sv, torch, oracle, dev, stream, with_cpu=not args.no_cpu)
    sts = None if args.no_sts else sts_leg(sv, torch, oracle, dev, stream, with_cpu=not args.no_cpu)

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("workload") == args.config and tj.get("kernel_source_sha") == _kernel_sha():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, oracle, args.cpu_seconds, L, args.pool)
    props = torch.cuda.get_device_properties(dev)

    line = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: B={B} gamma={G} V={V} {w.dtype} logits ({recipe(args.config)}), "
                               f"schedule (budget {w.budget} tokens, early stop) + verify of the selected "
                               f"prefixes",
                   "B": B, "gamma": G, "V": V, "budget_tokens": w.budget,
                   "scheduled_positions": positions, "rows_streamed": rows,
                   "verification": ("left to right, stopping at the first rejection (two streaming passes)"
                                    if ltr else "every scheduled position"),
                   "rows_scheduled": rows_scheduled},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "frac_scope": "the row-streaming kernel alone; path_frac covers the whole step",
                     "path_achieved": path_gbps, "path_frac": path_gbps / PEAK_HBM_GBS,
                     "kernel": "stream_kernel<bf16>", "ms_per_launch": ms_stream,
                     "ms_per_launch_median": ms_stream_median,
                     "timed_launches": 0 if greedy else len(per_launch),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": achieved / ceiling["gbps"]},
        "cpu_baseline": cpu,
        "left_to_right": walk,
        "overlap_mass": overlap,
        "async_scheduler": async_sched,
        "draft_sampler": draft,
        "temperature_scaling": sts,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory},
        "ms_breakdown": {"stream_kernel": ms_stream, "rest_of_step": ms_step - ms_stream},
    }
    print(json.dumps(line), flush=True)


def recipe(name):
    """The workload's logit recipe in words (the generator's parameters)."""
    from workloads import CONFIGS
    c = CONFIGS[name]
    t = f"target N(0,{c['target_std']:g})" + (f" + {c['spike']:g} on one token per row" if c["spike"] else "")
    nz = c["noise"]
    if nz is None:
        d = "no draft logits"
    elif nz[0] == "const":
        d = f"draft = target + N(0,{nz[1]:g})"
    else:
        d = f"draft_k = target_k + N(0,{nz[1]:g}+{nz[2]:g}k)"
    return f"{t}, {d}"


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("verify.hip", "verify_impl.hpp", "common.hpp", "philox.hpp"):
        p = os.path.join(ROOT, "draft_verification_04_amd", "csrc", f)
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_ceiling(sv, torch, copies, nbytes, stream, reps=20):
    """Best rate of spec_read_ceiling (a plain 16-byte read kernel) over `nbytes` of the logits,
    alternating the input copies as the timed steps do, over grid sizes up to a few vectors per
    thread (the largest grids read fastest on this device)."""
    from draft_verification_04_amd.hipevents import HipEvent
    dev = copies[0][0].device
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    src = [c[0] for c in copies]
    if src[0].numel() * src[0].element_size() < nbytes:  # more bytes than the target rows hold
        src = [torch.empty(nbytes + 16, dtype=torch.uint8, device=dev) for _ in range(len(copies))]
    best = None
    for grid in (2048, 4096, 8192, 16384, 32768):
        for r in range(2):   # warm-up
            sv.read_ceiling(src[r % len(src)], nbytes, grid, sink, stream)
        e0, e1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for r in range(reps):
            sv.read_ceiling(src[r % len(src)], nbytes, grid, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_ms(e1) / reps
        gbps = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": gbps, "ms": ms, "grid": grid, "bytes": nbytes, "kernel": "spec_read_ceiling"}
    return best


def ltr_first_pass(G, V, elem_bytes):
    """Positions the first pass of a left-to-right call streams (the library's own answer)."""
    import draft_verification_04_amd as sv
    return int(sv.load_library().spec_left_to_right_first_pass(G, V, 1 if elem_bytes == 2 else 0))


def ltr_rows(L, n_acc, G, cap):
    """Rows the two passes of a left-to-right call read: positions 0 .. cap-1 of every request (both
    rows of a draft position, the target row alone at k = L), then positions cap .. L of the requests
    whose walk passed every one of those (accepted length >= cap; the bench's rows are all valid)."""
    L = np.asarray(L, dtype=np.int64)
    n_acc = np.asarray(n_acc, dtype=np.int64)
    first = np.minimum(L + 1, cap)
    rows1 = 2 * np.minimum(first, L) + (first > L)
    more = (L >= cap) & (n_acc >= cap)
    return int(rows1.sum() + np.where(more, 2 * (L - cap) + 1, 0).sum())


def ltr_leg(sv, torch, w, copies, sps, ws, sch_ws, stream, ms_full, L, reps=200):
    """The same step as spec_schedule_verify with SPEC_VERIFY_LEFT_TO_RIGHT (DSpark paper §2.1: the
    walk stops at the first rejection, so rows after it are not read; accept_prob is NaN after it).
    Two streaming passes, positions 0 .. c-1 of every request (c = ltr_first_pass), then positions
    c .. L of the requests whose walk passed all of them; HIP events around the whole loop and around
    the two passes of every tenth call.  Not the headline step."""
    from draft_verification_04_amd.hipevents import HipEvent
    B, G = w.B, w.gamma
    dev = w.target.device
    out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
               out_tokens=torch.empty((B, G + 1), dtype=torch.int32, device=dev),
               accept_prob=torch.empty((B, G), dtype=torch.float32, device=dev),
               status=torch.empty(B, dtype=torch.int32, device=dev),
               lengths=torch.empty(B, dtype=torch.int32, device=dev),
               theta=torch.empty(1, dtype=torch.float64, device=dev),
               sched_status=torch.empty(B, dtype=torch.int32, device=dev))

    def call(r, events=None):
        tgt, drf = copies[r % len(copies)]
        sv.schedule_verify(tgt, drf, w.draft_tokens, w.conf, sps, w.budget, sv.SPEC_SCHED_EARLY_STOP,
                           w.temperature, w.top_k, w.seed, out=out, workspace=ws, sched_workspace=sch_ws,
                           stream=stream, events=events, left_to_right=True)
    for r in range(100):   # the headline step's warm-up
        call(r)
    evs = [(HipEvent(), HipEvent()) if r % 10 == 0 else None for r in range(reps)]
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for r in range(reps):
        call(r, evs[r])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    ms_passes = float(np.mean([e[0].elapsed_ms(e[1]) for e in evs if e is not None]))
    rows = ltr_rows(L, out["num_accepted"].cpu().numpy(), G, ltr_first_pass(G, w.V, w.elem_bytes))
    row_bytes = w.V * w.elem_bytes
    pos = int(np.asarray(L).sum())
    return {"ms_per_step": ms, "positions_per_s": pos / (ms * 1e-3), "vs_full_step": ms_full / ms,
            "rows_streamed": rows, "rows_scheduled": int((2 * np.asarray(L) + 1).sum()),
            "ms_two_passes": ms_passes,
            "gbps_two_passes": rows * row_bytes / (ms_passes * 1e-3) / 1e9,
            "note": "first pass start to second pass end, the walk kernel between them included"}


def overlap_leg(sv, torch, w, copies, lengths, stream, reps=20):
    """spec_overlap_mass (per-position sum_v min(p_t, p_d)) on the same workload and lengths,
    timed with HIP events; not part of the step.  Each draft position's row pair is read twice
    (statistics, then the overlap)."""
    from draft_verification_04_amd.hipevents import HipEvent
    B, G = w.B, w.gamma
    out = dict(overlap=torch.empty((B, G), dtype=torch.float64, device=w.target.device),
               status=torch.empty(B, dtype=torch.int32, device=w.target.device))
    ws = torch.empty(sv.load_library().spec_overlap_workspace_size(B, G, w.V), dtype=torch.uint8,
                     device=w.target.device)
    call = lambda r: sv.overlap_mass(copies[r % len(copies)][0], copies[r % len(copies)][1], lengths,
                                     w.temperature, w.top_k, out=out, workspace=ws, stream=stream)
    for r in range(2):
        call(r)
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for r in range(reps):
        call(r)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    pos = int(lengths.sum().item()) if lengths is not None else w.B * w.gamma
    row_bytes = w.V * w.elem_bytes
    once = 2 * pos * row_bytes
    return {"ms_per_call": ms, "positions": pos, "positions_per_s": pos / (ms * 1e-3),
            "rows_per_pass": 2 * pos, "bytes_read_per_call": 2 * once,
            "gbps_read": 2 * once / (ms * 1e-3) / 1e9, "algorithmic_bytes_once": once}


def draft_leg(sv, torch, oracle, dev, stream, reps=10, with_cpu=True):
    """spec_draft_markov (the Markov-head sequential sampler and the confidence head) on the
    draft block of the same shape: B=256 requests, gamma=16, V=151936, r=256, hidden size 4096,
    bf16, temperatures U[0.6, 1.2] with every fifth request greedy; HIP events around whole calls.
    Not part of the step (the verifier's input is the drafter's output)."""
    from draft_verification_04_amd.hipevents import HipEvent
    from workloads import make_draft_inputs
    B, G, V, r, d = 256, 16, 151936, 256, 4096
    w = make_draft_inputs(B, G, V, r, d, "bf16", "gaussian", "mixed", 2024, dev)
    out = dict(tokens=torch.empty((B, G), dtype=torch.int32, device=dev), logits=torch.empty_like(w.base),
               conf=torch.empty((B, G), dtype=torch.float32, device=dev),
               status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = torch.empty(sv.load_library().spec_draft_workspace_size(B, G, V), dtype=torch.uint8, device=dev)
    call = lambda: sv.draft_markov(w.base, w.W1, w.W2t, w.anchor, w.temperature, w.seed, w.hidden, w.conf_w,
                                   out=out, workspace=ws, stream=stream)
    for _ in range(2):
        call()
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    nwg = (V + 127) // 128
    step_bytes = 2 * B * V * 2 + V * r * 2 + B * r * 2 + B * nwg * 8    # U_k in, z_k out, W2, W1 rows, tiles
    sample_bytes = B * V * 2 + B * nwg * 8                               # the sampler reads z_k and the tiles
    flops = 2.0 * B * V * r * G
    res = {"config": f"B={B} gamma={G} V={V} r={r} d={d} bf16", "ms_per_call": ms,
           "draft_tokens_per_s": B * G / (ms * 1e-3), "status_ok": int((out["status"] == 0).sum().item()),
           "bytes_per_step_kernel": step_bytes, "bytes_per_step_sampler": sample_bytes,
           "gbps_per_call": G * (step_bytes + sample_bytes) / (ms * 1e-3) / 1e9,
           "mfma_tflops_per_call": flops / (ms * 1e-3) / 1e12}
    if with_cpu:
        from threadpoolctl import threadpool_limits
        sample = [0, 1]
        with threadpool_limits(1):
            t0 = time.perf_counter()
            n = len(sample)   # the first requests of the batch, as a slice (the oracle's outputs are per row)
            oracle.markov_draft(w.base[:n], w.W1.cpu(), w.W2t.cpu(), w.anchor[:n].cpu(), w.temperature[:n].cpu(),
                                w.seed[:n].cpu(), w.hidden[:n], w.conf_w.cpu())
            el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(sample) * G / el, "unit": "draft tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"requests {sample} x {G} positions, numpy fp64, one BLAS thread, "
                                         f"{el:.1f} s"}
    del w, out, ws
    torch.cuda.empty_cache()
    return res


def sts_leg(sv, torch, oracle, dev, stream, reps=3, with_cpu=True):
    """spec_sts_fit (Sequential Temperature Scaling) on 2^20 held-out instances x 16 positions with
    a 256-value temperature grid and 15 bins; HIP events around whole fits.  One evaluation = one
    (instance, position, grid value): a sigmoid, a product and a bin update, all fp64."""
    from draft_verification_04_amd.hipevents import HipEvent
    from workloads import make_sts_inputs, tau_grid
    N, G, T = 1 << 20, 16, 256
    t, y, kappa = make_sts_inputs(N, G, 11, device=dev)
    taus = tau_grid(T, device=dev)
    ws = torch.empty(sv.load_library().spec_sts_workspace_size(N, T, 15), dtype=torch.uint8, device=dev)
    out = sv.sts_fit(t, y, taus, 15, workspace=ws, stream=stream)
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        sv.sts_fit(t, y, taus, 15, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    evals = N * G * T
    res = {"config": f"N={N} gamma={G} grid={T} bins=15", "ms_per_fit": ms, "evaluations_per_s": evals / (ms * 1e-3),
           "tau": [round(float(v), 4) for v in out["tau"].cpu().tolist()],
           "kappa_synthetic": [round(float(v), 4) for v in kappa]}
    if with_cpu:
        from threadpoolctl import threadpool_limits
        n_cpu = 1 << 16
        with threadpool_limits(1):
            t0 = time.perf_counter()
            oracle.sts_fit(t[:n_cpu, :2].cpu().numpy(), y[:n_cpu, :2].cpu().numpy(), taus.cpu().numpy(), 15)
            el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n_cpu * 2 * T / el, "unit": "evaluations/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n_cpu} instances x 2 positions x {T} grid values, numpy fp64, one "
                                         f"BLAS thread, {el:.1f} s"}
    return res


def async_scheduler_leg(sv, torch, w, sps, stream, reps=20):
    """The asynchronous scheduler of the same workload: spec_schedule_capacity (the global search,
    off the critical path in a pipeline) and spec_schedule_topk (the per-step top-K admission),
    each timed with HIP events; the synchronous early-stop scheduler of the step for comparison."""
    from draft_verification_04_amd.hipevents import HipEvent
    ws = torch.empty(max(256, sv.load_library().spec_schedule_workspace_size(w.B, w.gamma)), dtype=torch.uint8,
                     device=w.conf.device)
    cap = sv.schedule_capacity(w.conf, sps, w.budget, stream=stream, workspace=ws)
    top = sv.schedule_topk(w.conf, cap["capacity"], stream=stream, workspace=ws)
    sync = sv.schedule_lengths(w.conf, sps, w.budget, stream=stream, workspace=ws)

    def timed(fn):
        fn()
        e0, e1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / reps

    t_cap = timed(lambda: sv.schedule_capacity(w.conf, sps, w.budget, out=cap, stream=stream, workspace=ws))
    t_top = timed(lambda: sv.schedule_topk(w.conf, cap["capacity"], out=top, stream=stream, workspace=ws))
    t_es = timed(lambda: sv.schedule_lengths(w.conf, sps, w.budget, out=sync, stream=stream, workspace=ws))
    return {"capacity_ms": t_cap, "topk_ms": t_top, "early_stop_ms": t_es,
            "capacity": int(cap["capacity"].item()), "topk_positions": int(top["lengths"].sum().item()),
            "early_stop_positions": int(sync["lengths"].sum().item())}


_POOL = {}


def _pool_verify(req):
    d = _POOL
    out = d["oracle"].verify(d["target"], d["draft"], d["tokens"], d["lengths"], d["temperature"], d["top_k"],
                             d["seed"], requests=req)
    return int(out["num_accepted"][req].size)


def cpu_baseline(w, oracle, budget_s, L, pool):
    """Time the oracle on the same workload: single-threaded on the first requests until the
    budget is spent, then over all requests with a pool of forked worker processes."""
    conf = w.conf.cpu().numpy() if w.conf is not None else None
    t_start = time.perf_counter()
    if conf is not None:
        oracle.schedule(conf, w.sps, w.budget)
    t_sched = time.perf_counter() - t_start
    done = 0
    positions = 0
    t0 = time.perf_counter()
    chunk = 4
    while time.perf_counter() - t0 < budget_s and done < w.B:
        req = list(range(done, min(w.B, done + chunk)))
        oracle.verify(w.target, w.draft, w.draft_tokens,
                      None if conf is None else L, w.temperature, w.top_k, w.seed, requests=req)
        positions += int(L[req].sum())
        done += len(req)
    el = time.perf_counter() - t0
    # the scheduler runs once per step for the whole batch: charge it pro rata
    el_total = el + t_sched * done / w.B
    single = positions / el_total
    # pooled: host copies once (bf16 -> fp32 is exact), workers forked with them; the workers
    # only run numpy and exit without touching the GPU
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    n = max(1, min(pool if pool > 0 else 16, affinity))
    Lh = np.asarray(L)
    _POOL.update(oracle=oracle, target=w.target.float().cpu().numpy(), draft=w.draft.float().cpu().numpy(),
                 tokens=w.draft_tokens.cpu().numpy(), lengths=Lh,
                 temperature=w.temperature.cpu().numpy() if w.temperature is not None else None,
                 top_k=w.top_k.cpu().numpy() if w.top_k is not None else None,
                 seed=w.seed.cpu().numpy() if w.seed is not None else None)
    chunks = [list(range(a, min(w.B, a + 4))) for a in range(0, w.B, 4)]
    ctx = mp.get_context("fork")
    with ctx.Pool(n) as p:
        t0 = time.perf_counter()
        p.map(_pool_verify, chunks, chunksize=1)
        el_pool = time.perf_counter() - t0
    _POOL.clear()
    pooled = int(Lh.sum()) / (el_pool + t_sched)
    return {"value": pooled, "unit": "positions/s", "cores": n, "kind": "oracle", "host_affinity_cores": affinity,
            "sample": f"all {w.B} requests ({int(Lh.sum())} verified positions) over {n} forked numpy fp64 "
                      f"worker processes (of {affinity} host cores in this process's affinity) in "
                      f"{el_pool:.1f} s, plus the scheduler ({t_sched:.2f} s, one thread)",
            "single_thread": {"value": single, "cores": 1,
                              "sample": f"first {done} of {w.B} requests ({positions} verified positions), "
                                        f"verify {el:.1f} s + scheduler {t_sched:.2f} s pro rata"}}


if __name__ == "__main__":
    main()
