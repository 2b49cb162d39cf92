"""spec_verify_static (the entry point for callers that cannot allocate) against spec_verify,
through the C ABI: two calls in a row on one stream, the second with a smaller input, each
compared with spec_verify's outputs on the same inputs bit for bit (the two share every kernel;
only the workspace differs).  A shape whose workspace exceeds the static array is refused
before any HIP call."""

import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from parity import HostInputs, compare_verify, run_oracle_pooled
from workloads import make_workload

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_04_amd as m
    m.load_library()
    return m


def _outs(B, G):
    return dict(num_accepted=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                out_tokens=torch.full((B, G + 1), -7, dtype=torch.int32, device=DEV),
                accept_prob=torch.full((B, G), -7.0, dtype=torch.float32, device=DEV),
                status=torch.full((B,), -7, dtype=torch.int32, device=DEV))


def _static_call(sv, w, L, out, stream):
    """spec_verify_static through ctypes, every argument a raw pointer."""
    lib = sv.load_library()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dt = sv.SPEC_BF16 if w.target.dtype == torch.bfloat16 else sv.SPEC_F32
    return lib.spec_verify_static(w.B, w.gamma, w.V, dt, p(w.target), p(w.draft), p(w.draft_tokens), p(L),
                                  p(w.temperature), p(w.top_k), p(w.seed), p(out["num_accepted"]),
                                  p(out["out_tokens"]), p(out["accept_prob"]), p(out["status"]),
                                  ctypes.c_void_p(stream.cuda_stream))


def _same(a, b):
    for k in ("num_accepted", "out_tokens", "status"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["accept_prob"].view(torch.int32), b["accept_prob"].view(torch.int32))


def test_two_calls_in_a_row_match_spec_verify(sv):
    stream = torch.cuda.current_stream()
    big = make_workload("mixed", DEV, B=300, gamma=8, V=129280, seed=81)     # the fused emit, top-k
    small = make_workload("mid", DEV, B=24, gamma=5, V=20011, seed=82)       # the split emit, odd V
    rng = np.random.default_rng(83)
    Ls = [torch.from_numpy(rng.integers(0, w.gamma + 1, w.B).astype(np.int32)).to(DEV) for w in (big, small)]
    got = []
    for w, L in zip((big, small), Ls):
        print(f"case B={w.B} gamma={w.gamma} V={w.V}", flush=True)
        out = _outs(w.B, w.gamma)
        assert _static_call(sv, w, L, out, stream) == sv.SPEC_OK
        got.append(out)
    torch.cuda.synchronize()
    for w, L, out in zip((big, small), Ls, got):
        ref = sv.verify(w.target, w.draft, w.draft_tokens, L, w.temperature, w.top_k, w.seed)
        torch.cuda.synchronize()
        _same(out, ref)
        h = HostInputs.of_workload(w, L)
        compare_verify(out, run_oracle_pooled(h), inputs=h)


def test_the_binding_and_a_repeat_on_the_larger_shape(sv):
    # the array keeps the last call's contents: a larger call after a smaller one must not read them
    stream = torch.cuda.current_stream()
    w = make_workload("scheduled", DEV, B=256, gamma=16, V=151936, seed=84)
    out = _outs(w.B, w.gamma)
    sv.verify_static(w.target, w.draft, w.draft_tokens, None, w.temperature, w.top_k, w.seed, out=out,
                     stream=stream)
    ref = sv.verify(w.target, w.draft, w.draft_tokens, None, w.temperature, w.top_k, w.seed)
    torch.cuda.synchronize()
    _same(out, ref)


def test_too_large_a_shape_is_refused(sv):
    lib = sv.load_library()
    B, G, V = 4096, 64, 524288
    assert lib.spec_verify_workspace_size(B, G, V) > 128 << 20
    z = torch.zeros(16, dtype=torch.int32, device=DEV)
    p = ctypes.c_void_p(z.data_ptr())
    assert lib.spec_verify_static(B, G, V, 1, p, p, p, None, p, None, p, p, p, None, None, None) == sv.SPEC_ERR_WORKSPACE


def test_static_call_replayed_from_a_captured_graph(sv):
    """The use the entry point is for: spec_verify_static recorded into a HIP graph (no allocation,
    no memset node: the kernels write every workspace word they read) and replayed three times,
    with eager work between the replays; every replay's outputs equal the eager call's bit for bit.
    The first eager call looks the array's address up, outside the capture."""
    w = make_workload("mixed", DEV, B=256, gamma=6, V=30011, seed=91)   # the fused emit, top-k
    L = torch.from_numpy(np.random.default_rng(92).integers(0, 7, 256).astype(np.int32)).to(DEV)
    s = torch.cuda.Stream()
    ref = _outs(w.B, w.gamma)
    with torch.cuda.stream(s):
        assert _static_call(sv, w, L, ref, s) == 0
    s.synchronize()
    out = _outs(w.B, w.gamma)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        code = _static_call(sv, w, L, out, s)
    assert code == 0
    other = make_workload("mid", DEV, B=16, gamma=3, V=5003, seed=93)
    for rep in range(3):
        for t in out.values():
            t.fill_(-7)                      # a fill kernel, between the replays
        sv.verify(other.target, other.draft, other.draft_tokens, None, other.temperature, None, other.seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        _same(out, ref)
