"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments synchronously before touching the device."""

import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "spec_verify.h")
LIB = os.path.join(ROOT, "draft_verification_04_amd", "libspecverify.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspecverify.so is not built (run __graft_entry__.build())")
    import draft_verification_04_amd as sv
    return sv.load_library()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("spec_verify", "spec_verify_greedy", "spec_schedule_lengths", "spec_verify_workspace_size",
              "spec_schedule_workspace_size", "spec_abi_version", "spec_status_string",
              "spec_philox_uniforms", "spec_verify_profiled", "spec_verify_greedy_workspace_size",
              "spec_read_ceiling", "spec_left_to_right_first_pass", "spec_verify_flat", "spec_overlap_mass", "spec_schedule_capacity",
              "spec_schedule_topk", "spec_draft_markov", "spec_draft_workspace_size", "spec_sts_fit",
              "spec_sts_apply", "spec_sts_workspace_size", "spec_verify_bounded"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b[TW] (spec_\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        getattr(lib, n)


def test_binding_covers_every_symbol(lib):
    import draft_verification_04_amd as sv
    assert set(sv.EXPORTS) == set(_declared())


def test_version_and_strings(lib):
    assert lib.spec_abi_version() == 3
    for code, text in ((0, "ok"), (1, "invalid argument"), (2, "workspace"), (3, "unsupported"), (4, "HIP")):
        assert text in lib.spec_status_string(code).decode()
    assert lib.spec_status_string(99).decode() == "unknown status"


def test_left_to_right_first_pass(lib):
    assert lib.spec_left_to_right_first_pass(16, 151936, 1) == 3     # rows of 6 segments
    assert lib.spec_left_to_right_first_pass(2, 151936, 1) == 2      # at most gamma
    assert lib.spec_left_to_right_first_pass(1, 1000, 0) == 1
    assert lib.spec_left_to_right_first_pass(16, 262144, 1) == 2     # rows of 10 segments
    assert lib.spec_left_to_right_first_pass(16, 196608, 1) == 3     # exactly 8 segments
    assert lib.spec_left_to_right_first_pass(16, 196608, 0) == 2     # fp32: 16 segments
    assert lib.spec_left_to_right_first_pass(0, 1000, 1) == 0
    assert lib.spec_left_to_right_first_pass(16, 0, 1) == 0
    assert lib.spec_left_to_right_first_pass(16, 1000, 7) == 0


def test_workspace_sizes(lib):
    a = lib.spec_verify_workspace_size(256, 16, 151936)
    b = lib.spec_verify_workspace_size(512, 16, 151936)
    assert 0 < a < b and a % 256 == 0
    assert lib.spec_verify_workspace_size(0, 16, 10) == 0
    assert lib.spec_verify_workspace_size(4, 65, 10) == 0
    assert lib.spec_verify_greedy_workspace_size(4, 8) > 0
    assert lib.spec_schedule_workspace_size(256, 16) >= 12 * 256 * 16


def _fake(n=64):
    # Host buffers standing in for device pointers: validation must reject the call before any
    # of them is dereferenced.  The address is 16-byte aligned (as logits must be) but never
    # 256-byte aligned, so used as a workspace it is always refused and nothing is launched.
    buf = (ctypes.c_uint8 * (n + 512))()
    addr = ((ctypes.addressof(buf) + 255) & ~255) + 16
    return buf, ctypes.c_void_p(addr)


def test_verify_rejects_bad_arguments_before_launch(lib):
    keep, p = _fake()
    ws = lib.spec_verify_workspace_size(2, 4, 100)
    base = dict(B=2, G=4, V=100, dt=1, t=p, d=p, x=p, L=None, T=p, K=None, s=p, n=p, o=p, r=None, st=None,
                ws=p, wsb=ws, stream=None)

    def call(**kw):
        a = dict(base, **kw)
        return lib.spec_verify(a["B"], a["G"], a["V"], a["dt"], a["t"], a["d"], a["x"], a["L"], a["T"], a["K"],
                               a["s"], a["n"], a["o"], a["r"], a["st"], a["ws"], a["wsb"], a["stream"])

    assert call(B=0) == 1
    assert call(G=0) == 1
    assert call(G=65) == 1
    assert call(V=0) == 1
    assert call(V=524289) == 1
    assert call(dt=0, V=262145) == 1
    assert call(dt=7) == 1
    assert call(t=None) == 1
    assert call(d=None) == 1
    assert call(x=None) == 1
    assert call(T=None) == 1
    assert call(s=None) == 1
    assert call(n=None) == 1
    assert call(o=None) == 1
    assert call(t=ctypes.c_void_p(p.value + 2)) == 1          # misaligned logits
    assert call(ws=None) == 2
    assert call(wsb=ws - 1) == 2
    assert call(ws=ctypes.c_void_p(p.value + 16)) == 2        # workspace not 256-byte aligned


def test_greedy_and_schedule_reject_bad_arguments(lib):
    keep, p = _fake()
    ws = lib.spec_verify_greedy_workspace_size(2, 4)
    assert lib.spec_verify_greedy(0, 4, 10, 1, p, p, None, p, p, None, p, ws, None) == 1
    assert lib.spec_verify_greedy(2, 4, 10, 1, None, p, None, p, p, None, p, ws, None) == 1
    assert lib.spec_verify_greedy(2, 4, 10, 1, p, p, None, p, p, None, None, ws, None) == 2
    # B, gamma, conf, sps, sps_len, budget, mode, lengths, theta, status, ws, wsb, stream
    assert lib.spec_schedule_lengths(0, 4, p, p, 100, 10, 0, p, None, None, None, 0, None) == 1
    assert lib.spec_schedule_lengths(4, 65, p, p, 100, 10, 0, p, None, None, None, 0, None) == 1
    assert lib.spec_schedule_lengths(4, 4, p, p, 100, 10, 2, p, None, None, None, 0, None) == 1
    assert lib.spec_schedule_lengths(4, 4, None, p, 100, 10, 0, p, None, None, None, 0, None) == 1
    assert lib.spec_schedule_lengths(4, 4, p, p, 10, 10, 0, p, None, None, None, 0, None) == 1   # table short
    assert lib.spec_schedule_lengths(4, 4, p, p, 4, 2, 0, p, None, None, None, 0, None) == 1     # needs sps[B]
    assert lib.spec_schedule_lengths(2048, 16, p, p, 10 ** 6, 10, 0, p, None, None, None, 0, None) == 3
    # valid shapes, no workspace
    assert lib.spec_schedule_lengths(4, 4, p, p, 100, 10, 0, p, None, None, None, 0, None) == 2
    n = lib.spec_schedule_workspace_size(256, 16)
    assert n >= 12 * 256 * 16 and n % 256 == 0 and lib.spec_schedule_workspace_size(0, 16) == 0
    assert lib.spec_schedule_lengths(4, 4, p, p, 100, 10, 0, p, None, None, p, 8, None) == 2   # short
    assert lib.spec_philox_uniforms(-1, p, p, p, p, p, None) == 1
    assert lib.spec_philox_uniforms(0, None, None, None, None, None, None) == 0


def test_read_ceiling_rejects_bad_arguments(lib):
    keep, p = _fake()
    assert lib.spec_read_ceiling(None, 1024, 64, p, None) == 1
    assert lib.spec_read_ceiling(ctypes.c_void_p(p.value + 4), 1024, 64, p, None) == 1   # misaligned
    assert lib.spec_read_ceiling(p, 8, 64, p, None) == 1
    assert lib.spec_read_ceiling(p, 1024, 0, p, None) == 1
    assert lib.spec_read_ceiling(p, 1024, 64, None, None) == 1


def test_overlap_rejects_bad_arguments(lib):
    keep, p = _fake()
    ws = lib.spec_overlap_workspace_size(2, 4, 10)
    assert ws > 0 and ws % 256 == 0 and lib.spec_overlap_workspace_size(0, 4, 10) == 0

    def call(B=2, G=4, V=10, dt=1, t=p, d=p, T=p, o=p, w=p, wsb=ws):
        return lib.spec_overlap_mass(B, G, V, dt, t, d, None, T, None, o, None, w, wsb, None)
    assert call(B=0) == 1
    assert call(G=65) == 1
    assert call(dt=7) == 1
    assert call(t=None) == 1
    assert call(T=None) == 1
    assert call(o=None) == 1
    assert call(d=ctypes.c_void_p(p.value + 2)) == 1
    assert call(w=None) == 2
    assert call(wsb=ws - 1) == 2


def test_async_scheduler_rejects_bad_arguments(lib):
    keep, p = _fake()
    assert lib.spec_schedule_capacity(0, 4, p, p, 100, 10, p, None, None, p, 4096, None) == 1
    assert lib.spec_schedule_capacity(4, 4, None, p, 100, 10, p, None, None, p, 4096, None) == 1
    assert lib.spec_schedule_capacity(4, 4, p, p, 100, 10, None, None, None, p, 4096, None) == 1
    assert lib.spec_schedule_capacity(4, 4, p, p, 10, 10, p, None, None, p, 4096, None) == 1   # table short
    assert lib.spec_schedule_capacity(2048, 16, p, p, 10 ** 6, 10, p, None, None, p, 4096, None) == 3
    assert lib.spec_schedule_capacity(4, 4, p, p, 100, 10, p, None, None, p, 4096, None) == 2   # workspace
    assert lib.spec_schedule_topk(0, 4, p, p, p, None, p, 4096, None) == 1
    assert lib.spec_schedule_topk(4, 65, p, p, p, None, p, 4096, None) == 1
    assert lib.spec_schedule_topk(4, 4, None, p, p, None, p, 4096, None) == 1
    assert lib.spec_schedule_topk(4, 4, p, None, p, None, p, 4096, None) == 1
    assert lib.spec_schedule_topk(4, 4, p, p, None, None, p, 4096, None) == 1
    assert lib.spec_schedule_topk(4, 4, p, p, p, None, p, 4096, None) == 2                  # workspace


def test_verify_flat_requires_lengths(lib):
    keep, p = _fake()
    ws = lib.spec_verify_workspace_size(2, 4, 100)
    # B, gamma, V, dtype, target_rows, n_target_rows, draft_rows, n_draft_rows, tokens, lengths, T, top_k,
    # seed, n, out_tokens, accept_prob, status, ws, ws_bytes, stream
    args = [2, 4, 100, 1, p, 10, p, 8, p, p, p, None, p, p, p, None, None, p, ws, None]
    assert lib.spec_verify_flat(*args) == 2                      # fake workspace is refused
    bad = list(args); bad[9] = None
    assert lib.spec_verify_flat(*bad) == 1                       # no lengths
    bad = list(args); bad[6] = ctypes.c_void_p(p.value + 2)
    assert lib.spec_verify_flat(*bad) == 1                       # misaligned rows
    bad = list(args); bad[5] = -1
    assert lib.spec_verify_flat(*bad) == 1                       # negative row count
    bad = list(args); bad[7] = -1
    assert lib.spec_verify_flat(*bad) == 1


def test_launch_size_bound(lib):
    """A call whose streaming grid would pass 2^32 work-items (one 512-thread workgroup per row
    pair and ~48 KB segment) is refused with SPEC_ERR_UNSUPPORTED before anything is enqueued,
    here with a host buffer as every pointer (a launch would fault on it)."""
    keep, p = _fake()
    big = (500000, 16, 1000, 0)          # ~66 GB of fp32 logits: fits in HBM, not in one grid
    ok = (250000, 15, 1000, 0)           # 4 M rows x 1 segment x 512 = 2^31 work-items
    for (B, G, V, dt), want in ((big, 3), (ok, 2)):
        args = [B, G, V, dt, p, p, p, None, p, None, p, p, p, None, None, p, 1 << 40, None]
        assert lib.spec_verify(*args) == want, (B, G, V)
        # the token cap sizes the grid: a small cap fits
        assert lib.spec_verify_bounded(*args, 4096, None, None) == (2 if B < 4194304 else 3)
    # the fused emit runs a 1024-thread workgroup per request: B >= 2^22 cannot launch
    args = [1 << 22, 1, 8, 1, p, p, p, None, p, None, p, p, p, None, None, p, 1 << 40, None]
    assert lib.spec_verify_bounded(*args, 16, None, None) == 3
    assert lib.spec_verify_greedy(500000, 16, 1000, 0, p, p, None, p, p, None, p, 1 << 40, None) == 3
    assert lib.spec_overlap_mass(500000, 16, 1000, 0, p, p, None, p, None, p, None, p, 1 << 40, None) == 3


def test_verify_bounded_rejects_a_bound_below_one(lib):
    keep, p = _fake()
    ws = lib.spec_verify_workspace_size(2, 4, 100)
    args = [2, 4, 100, 1, p, p, p, p, p, None, p, p, p, None, None, p, ws, None]
    assert lib.spec_verify_bounded(*args, 0, None, None) == 1
    assert lib.spec_verify_bounded(*args, -5, None, None) == 1
    assert lib.spec_verify_bounded(*args, 10, None, None) == 2   # a valid bound; fake workspace refused


def test_draft_rejects_bad_arguments(lib):
    keep, p = _fake()
    ws = lib.spec_draft_workspace_size(3, 4, 1000)
    assert ws > 0 and ws % 256 == 0 and lib.spec_draft_workspace_size(0, 4, 1000) == 0
    assert lib.spec_draft_workspace_size(3, 65, 1000) == 0

    def call(B=3, G=4, V=1000, r=256, dt=1, U=p, w1=p, w2=p, x0=p, T=p, d=0, h=None, cw=None,
             tok=p, z=p, conf=None, st=p, w=p, wsb=ws):
        return lib.spec_draft_markov(B, G, V, r, dt, U, w1, w2, x0, T, None, d, h, cw, None, tok, z, conf, st,
                                     w, wsb, None)
    assert call(w=None) == 2                       # every other argument is valid
    assert call(B=0) == 1
    assert call(G=0) == 1
    assert call(G=65) == 1
    assert call(r=8) == 1                          # rank not a multiple of 16
    assert call(r=264) == 1                        # rank above 256
    assert call(r=24) == 1
    assert call(dt=5) == 1
    assert call(U=None) == 1
    assert call(w2=None) == 1
    assert call(x0=None) == 1
    assert call(T=None) == 1
    assert call(tok=None) == 1
    assert call(st=None) == 1
    assert call(z=ctypes.c_void_p(p.value + 4)) == 1
    assert call(w1=ctypes.c_void_p(p.value + 8)) == 1
    assert call(conf=p) == 1                       # confidences without the head's weight
    assert call(conf=p, cw=p, d=16) == 1           # ... or without hidden states
    assert call(conf=p, cw=p, d=0) == 2            # d = 0 needs no hidden states
    assert call(d=-1) == 1
    assert call(wsb=ws - 1) == 2
    assert call(w=ctypes.c_void_p(p.value + 16)) == 2


def test_sts_rejects_bad_arguments(lib):
    keep, p = _fake()
    ws = lib.spec_sts_workspace_size(1000, 64, 15)
    assert ws > 0 and ws % 256 == 0
    assert lib.spec_sts_workspace_size(0, 64, 15) == 0 and lib.spec_sts_workspace_size(10, 64, 33) == 0

    def fit(N=1000, G=5, t=p, y=p, nt=64, tau=p, bins=15, out=p, w=p, wsb=ws):
        return lib.spec_sts_fit(N, G, t, y, nt, tau, bins, out, None, None, w, wsb, None)
    assert fit(w=None) == 2                        # every other argument is valid
    assert fit(N=0) == 1
    assert fit(G=65) == 1
    assert fit(nt=0) == 1
    assert fit(nt=5000) == 1
    assert fit(bins=0) == 1
    assert fit(bins=33) == 1
    assert fit(t=None) == 1
    assert fit(y=None) == 1
    assert fit(tau=None) == 1
    assert fit(out=None) == 1
    assert fit(wsb=ws - 1) == 2
    assert lib.spec_sts_apply(0, 4, p, p, p, None) == 1
    assert lib.spec_sts_apply(4, 65, p, p, p, None) == 1
    assert lib.spec_sts_apply(4, 4, None, p, p, None) == 1
    assert lib.spec_sts_apply(4, 4, p, None, p, None) == 1
    assert lib.spec_sts_apply(4, 4, p, p, None, None) == 1


def test_schedule_verify_rejects_bad_arguments(lib):
    keep, p = _fake()
    vws = lib.spec_verify_workspace_size(4, 4, 10)
    sws = lib.spec_schedule_workspace_size(4, 4)

    # every pointer argument defaults to the fake buffer; the workspaces are refused as misaligned
    def call(B=4, G=4, V=10, dt=1, conf=p, sps=p, sps_len=100, budget=10, mode=0, t=p, d=p, x=p, T=p, s=p,
             L=p, n=p, o=p, sw=p, swb=sws, vw=p, vwb=vws):
        return lib.spec_schedule_verify(B, G, V, dt, conf, sps, sps_len, budget, mode, t, d, x, T, None, s, L,
                                        None, None, n, o, None, None, sw, swb, vw, vwb, None, None, None)
    assert call(B=0) == 1
    assert call(G=65) == 1
    assert call(V=0) == 1
    assert call(dt=7) == 1
    assert call(mode=2) == 1
    assert call(budget=0) == 1
    assert call(sps_len=10) == 1                               # cost table short
    assert call(conf=None) == 1
    assert call(L=None) == 1
    assert call(t=None) == 1
    assert call(x=None) == 1
    assert call(s=None) == 1
    assert call(o=None) == 1
    assert call(d=ctypes.c_void_p(p.value + 2)) == 1           # misaligned logits
    assert call(B=2048, G=16, sps_len=10 ** 6) == 3
    assert call() == 2                                         # workspaces
    assert call(vwb=vws - 1) == 2
    # the left-to-right walk: refused up front outside 256 <= B <= 1024, gamma < 64, rows without
    # top-k and a budget of at least B (the fake workspaces would be refused after that check)
    ltr = 0x100
    assert call(mode=ltr) == 3                                  # B = 4
    assert call(mode=ltr | 1) == 3
    assert call(mode=ltr | 2) == 1                              # still a bad scheduler mode
    big = dict(B=256, G=16, V=1000, sps_len=10 ** 5, budget=2048)
    assert call(mode=ltr, **big) == 2                           # supported: reaches the workspaces
    assert call(mode=0, **big) == 2
    assert call(mode=ltr, **dict(big, budget=255)) == 3         # budget below B
    assert call(mode=ltr, **dict(big, B=1025, G=8, sps_len=10 ** 6, budget=4096)) == 3
    assert call(mode=0, **dict(big, B=1025, G=8, sps_len=10 ** 6, budget=4096)) == 2
    assert call(mode=ltr, **dict(big, G=64, sps_len=10 ** 6)) == 3
    assert lib.spec_schedule_verify(256, 16, 1000, 1, p, p, 10 ** 5, 2048, ltr, p, p, p, p, p, p, p, None, None,
                                    p, p, None, None, p, sws, p, vws, None, None, None) == 3   # top_k


def test_binding_refuses_host_tensors(lib):
    # the binding marshals device tensors only: host tensors are refused before any call
    import pytest
    import torch
    import draft_verification_04_amd as sv
    B, G, V = 2, 3, 16
    t = torch.zeros((B, G + 1, V))
    d = torch.zeros((B, G, V))
    x = torch.zeros((B, G), dtype=torch.int32)
    conf = torch.zeros((B, G))
    sps = torch.zeros(B * (G + 1) + 1, dtype=torch.float64)
    with pytest.raises(TypeError):
        sv.verify(t, d, x)
    with pytest.raises(TypeError):
        sv.schedule_verify(t, d, x, conf, sps, 4)
    with pytest.raises(TypeError):
        sv.schedule_lengths(conf, sps, 4)


def test_binding_checks_shapes_before_devices(lib):
    """Per-request vectors must hold B values and `out` tensors the shapes and dtypes the kernels
    write: the binding raises ValueError before any device check (host tensors suffice here)."""
    import torch
    import draft_verification_04_amd as sv
    B, G, V = 3, 4, 32
    t = torch.zeros((B, G + 1, V))
    d = torch.zeros((B, G, V))
    x = torch.zeros((B, G), dtype=torch.int32)
    L = torch.zeros(B, dtype=torch.int32)
    for kw in (dict(lengths=torch.zeros(B + 1, dtype=torch.int32)), dict(temperature=torch.ones(B - 1)),
               dict(top_k=torch.zeros((B, 1), dtype=torch.int32)), dict(seed=torch.zeros(2 * B, dtype=torch.int64))):
        with pytest.raises(ValueError):
            sv.verify(t, d, x, **kw)
    with pytest.raises(ValueError):
        sv.verify(t, d[:, :G - 1], x)
    with pytest.raises(ValueError):
        sv.verify(t, d, x[:, :G - 1])
    with pytest.raises(ValueError):
        sv.verify_greedy(t, x, lengths=torch.zeros(B - 1, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.verify_flat(t[0], d[0], x, None)                  # lengths define the layout
    with pytest.raises(ValueError):
        sv.verify_flat(t[0], d[0], x, torch.zeros(B + 2, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.verify_flat(t[0], d[0, :, :V - 1], x, L)
    with pytest.raises(ValueError):
        sv.overlap_mass(t, d, lengths=torch.zeros(B + 1, dtype=torch.int32))
    conf = torch.zeros((B, G))
    sps = torch.zeros(B * (G + 1) + 1, dtype=torch.float64)
    with pytest.raises(ValueError):
        sv.schedule_verify(t, d, x, conf[:, :G - 1], sps, 8)
    with pytest.raises(ValueError):
        sv.schedule_topk(conf, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.sts_apply(conf, torch.ones(G + 1, dtype=torch.float64))
    W = torch.zeros((V, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sv.draft_markov(d, W, W[:V - 1], torch.zeros(B, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.draft_markov(d, W, W, torch.zeros(B + 1, dtype=torch.int32))


def test_binding_checks_caller_outputs():
    """A caller's `out` tensors are checked for shape, dtype and device before the call."""
    import torch
    import draft_verification_04_amd as sv
    B, G, dev = 3, 4, torch.device("cpu")
    good = dict(num_accepted=torch.zeros(B, dtype=torch.int32), out_tokens=torch.zeros((B, G + 1), dtype=torch.int32),
                accept_prob=torch.zeros((B, G)), status=torch.zeros(B, dtype=torch.int32))
    spec = sv._verify_out_spec(B, G)
    assert sv._check_out(dict(good), spec, dev) is not None
    assert sv._check_out(dict(good, accept_prob=None, status=None), spec, dev) is not None   # optional
    for key, bad in (("out_tokens", torch.zeros((B, G), dtype=torch.int32)),
                     ("num_accepted", torch.zeros(B + 1, dtype=torch.int32)),
                     ("accept_prob", torch.zeros((B, G + 1))),
                     ("status", torch.zeros((B, 1), dtype=torch.int32))):
        with pytest.raises(ValueError):
            sv._check_out(dict(good, **{key: bad}), spec, dev)
    with pytest.raises(TypeError):
        sv._check_out(dict(good, out_tokens=torch.zeros((B, G + 1), dtype=torch.int64)), spec, dev)
    with pytest.raises(TypeError):
        sv._check_out(dict(good, accept_prob=torch.zeros((B, G), dtype=torch.float64)), spec, dev)
    with pytest.raises(ValueError):
        sv._check_out(dict(good, num_accepted=None), spec, dev)                   # required
    with pytest.raises(ValueError):
        sv._check_out(dict(good), spec, torch.device("meta"))                    # another device
