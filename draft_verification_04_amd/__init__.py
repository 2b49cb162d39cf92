"""Python binding of libspecverify: lossless draft verification on MI355X.

A thin ctypes layer over the C ABI declared in include/spec_verify.h.  It
only marshals arguments (torch CUDA tensors -> device pointers, the current
HIP stream, a workspace tensor); every step of the computation runs in the
library's HIP kernels.  If the library is missing the calls raise: there is
no CPU fallback.

    from draft_verification_04_amd import verify, verify_greedy, schedule_lengths
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK = 0
SPEC_ERR_INVALID_ARG = 1
SPEC_ERR_WORKSPACE = 2
SPEC_ERR_UNSUPPORTED = 3
SPEC_ERR_HIP = 4
SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_SCHED_EARLY_STOP = 0
SPEC_SCHED_GLOBAL = 1
SPEC_VERIFY_LEFT_TO_RIGHT = 0x100

REQ_BAD_TOKEN = 1
REQ_BAD_TEMPERATURE = 2
REQ_NONFINITE = 4
REQ_BAD_LENGTH = 8
REQ_BAD_TOPK = 16
REQ_BAD_CONFIDENCE = 32
REQ_OVER_BUDGET = 64
REQ_BAD_ROWS = 128

# name -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
EXPORTS = {
    "spec_abi_version": (_I, []),
    "spec_status_string": (ctypes.c_char_p, [_I]),
    "spec_verify_workspace_size": (_Z, [_I, _I, _I]),
    "spec_verify": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_verify_profiled": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P,
                                  _P, _P]),
    "spec_verify_bounded": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P,
                                 _I, _P, _P]),
    "spec_verify_static": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "spec_verify_flat": (_I, [_I, _I, _I, _I, _P, ctypes.c_int64, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P,
                              _P, _P, _P, _Z, _P]),
    "spec_verify_greedy_workspace_size": (_Z, [_I, _I]),
    "spec_verify_greedy": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_schedule_workspace_size": (_Z, [_I, _I]),
    "spec_schedule_lengths": (_I, [_I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "spec_schedule_verify": (_I, [_I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _Z, _P, _Z, _P, _P, _P]),
    "spec_philox_uniforms": (_I, [_I, _P, _P, _P, _P, _P, _P]),
    "spec_read_ceiling": (_I, [_P, _Z, _I, _P, _P]),
    "spec_left_to_right_first_pass": (_I, [_I, _I, _I]),
    "spec_overlap_workspace_size": (_Z, [_I, _I, _I]),
    "spec_schedule_capacity": (_I, [_I, _I, _P, _P, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "spec_schedule_topk": (_I, [_I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_overlap_mass": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_draft_workspace_size": (_Z, [_I, _I, _I]),
    "spec_draft_markov": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                               _Z, _P]),
    "spec_sts_workspace_size": (_Z, [_I, _I, _I]),
    "spec_sts_fit": (_I, [_I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, _Z, _P]),
    "spec_sts_apply": (_I, [_I, _I, _P, _P, _P, _P]),
}

_lib_handle = None


class SpecError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m draft_verification_04_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib_handle = lib
    return lib


def status_string(code: int) -> str:
    return load_library().spec_status_string(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _launch(stream, allocated, call):
    """Run call(hip_stream) on `stream` (default: the current stream) and return its code.

    The binding allocates and fills tensors (workspaces, default temperatures and seeds,
    outputs) on the current stream.  When `stream` is another stream it first waits for that
    work, and afterwards each tensor in `allocated` is marked as in use by it, so the caching
    allocator does not hand the memory to other work before the call's kernels are done with it.
    Tensors the caller passed in stay the caller's to order.
    """
    cur = torch.cuda.current_stream()
    s = cur if stream is None else stream
    side = s != cur
    if side:
        s.wait_stream(cur)
    code = call(ctypes.c_void_p(s.cuda_stream))
    if side:
        for t in allocated:
            if t is not None:
                t.record_stream(s)
    return code


def _check(fn, code):
    if code != SPEC_OK:
        raise SpecError(fn, code)


def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


def _vec(t, name, n):
    """A per-request vector must hold exactly n values (checked before the device checks)."""
    if t is not None and (not isinstance(t, torch.Tensor) or t.dim() != 1 or t.numel() != n):
        raise ValueError(f"{name} must be a 1-D tensor of {n} values")
    return t


def _shape(t, name, shape):
    if t is not None and (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape)):
        got = tuple(t.shape) if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")
    return t


def _check_out(out, spec, device):
    """Caller-supplied outputs: every tensor present must have the shape, dtype and device the
    kernels write (a missing optional one is passed as NULL)."""
    for key, (shape, dtype, required) in spec.items():
        t = out.get(key)
        if t is None:
            if required:
                raise ValueError(f"out[{key!r}] is required")
            continue
        _shape(t, f"out[{key!r}]", shape)
        if t.dtype != dtype:
            raise TypeError(f"out[{key!r}] has dtype {t.dtype}, expected {dtype}")
        if t.device != device or not t.is_contiguous():
            raise ValueError(f"out[{key!r}] must be a contiguous tensor on {device}")
    return out


def _on(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the logits on {device}")


def _logit_dtype(t):
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def verify_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return int(load_library().spec_verify_workspace_size(B, gamma, V))


def _workspace(nbytes: int, device, workspace=None, allocated=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if allocated is not None:
        allocated.append(ws)
    return ws


_SEED_DTYPES = (torch.int64, torch.uint64) if hasattr(torch, "uint64") else torch.int64


def _verify_inputs(target, draft, draft_tokens, lengths, temperature, top_k, seed):
    """Checks the verify inputs (shapes first, then device and dtype); returns
    (B, gamma, V, temperature, seed, allocated) with the defaults filled in."""
    if not isinstance(target, torch.Tensor) or target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    G = G1 - 1
    _shape(draft, "draft", (B, G, V))
    _shape(draft_tokens, "draft_tokens", (B, G))
    for name, t in (("lengths", lengths), ("temperature", temperature), ("top_k", top_k), ("seed", seed)):
        _vec(t, name, B)
    _dev(target, "target", (torch.float32, torch.bfloat16), 3)
    _dev(draft, "draft", target.dtype, 3)
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    _dev(lengths, "lengths", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    _dev(seed, "seed", _SEED_DTYPES, 1)
    dev = target.device
    _on(dev, draft=draft, draft_tokens=draft_tokens, lengths=lengths, temperature=temperature, top_k=top_k,
        seed=seed)
    allocated = []
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
        allocated.append(temperature)
    if seed is None:
        seed = torch.zeros(B, dtype=torch.int64, device=dev)
        allocated.append(seed)
    return B, G, V, temperature, seed, allocated


def _verify_out_spec(B, G):
    return dict(num_accepted=((B,), torch.int32, True), out_tokens=((B, G + 1), torch.int32, True),
                accept_prob=((B, G), torch.float32, False), status=((B,), torch.int32, False))


def _verify_outputs(B, G, dev, out, allocated):
    """A caller's `out` is checked and used as given (a missing accept_prob or status is passed as
    NULL); otherwise the outputs are allocated here."""
    if out is not None:
        return _check_out(out, _verify_out_spec(B, G), dev)
    out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
               out_tokens=torch.empty((B, G + 1), dtype=torch.int32, device=dev),
               accept_prob=torch.empty((B, G), dtype=torch.float32, device=dev),
               status=torch.empty(B, dtype=torch.int32, device=dev))
    allocated.extend(out.values())
    return out


def _events(events):
    if events is None:
        return None, None
    return ctypes.c_void_p(events[0].cuda_event), ctypes.c_void_p(events[1].cuda_event)


def verify(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
           lengths: Optional[torch.Tensor] = None, temperature: Optional[torch.Tensor] = None,
           top_k: Optional[torch.Tensor] = None, seed: Optional[torch.Tensor] = None,
           out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None,
           events=None, max_tokens: Optional[int] = None) -> dict:
    """spec_verify on torch tensors.  Returns dict(num_accepted, out_tokens, accept_prob, status).

    target [B, gamma+1, V] and draft [B, gamma, V] (float32 or bfloat16);
    draft_tokens [B, gamma] int32; lengths [B] int32 or None; temperature [B]
    float32 (default ones); top_k [B] int32 or None; seed [B] int64 holding
    the uint64 bit pattern (default zeros).  `events` = (before, after)
    HipEvent pair taking the start and end of the row-streaming kernel.
    `max_tokens` (spec_verify_bounded): the caller's bound on sum_i (L_i + 1),
    e.g. the scheduler's token budget; it sizes the streaming grid only.
    `stream`: a torch stream to enqueue on (default: the current stream).
    """
    lib = load_library()
    B, G, V, temperature, seed, mine = _verify_inputs(target, draft, draft_tokens, lengths, temperature, top_k,
                                                      seed)
    dev = target.device
    out = _verify_outputs(B, G, dev, out, mine)
    nbytes = int(lib.spec_verify_workspace_size(B, G, V))
    ws = _workspace(nbytes, dev, workspace, mine)
    ev0, ev1 = _events(events)

    def call(sp):
        args = (B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(lengths),
                _ptr(temperature), _ptr(top_k), _ptr(seed), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
                _ptr(out.get("accept_prob")), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(),
                sp)
        if max_tokens is None:
            return lib.spec_verify_profiled(*args, ev0, ev1)
        return lib.spec_verify_bounded(*args, int(max_tokens), ev0, ev1)
    _check("spec_verify", _launch(stream, mine, call))
    return out


def verify_static(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                  lengths: Optional[torch.Tensor] = None, temperature: Optional[torch.Tensor] = None,
                  top_k: Optional[torch.Tensor] = None, seed: Optional[torch.Tensor] = None,
                  out: dict = None, stream=None) -> dict:
    """spec_verify_static: spec_verify with the library's own device workspace (no allocation in
    the call).  `out` (num_accepted, out_tokens, and optionally accept_prob and status) and the
    temperature and seed tensors are required here, since the binding must not allocate either;
    calls that overlap in time on one GPU race (see the header)."""
    lib = load_library()
    if out is None or temperature is None or seed is None:
        raise ValueError("verify_static allocates nothing: pass out, temperature and seed")
    B, G, V, temperature, seed, mine = _verify_inputs(target, draft, draft_tokens, lengths, temperature, top_k,
                                                      seed)
    out = _verify_outputs(B, G, target.device, out, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_verify_static(
        B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(lengths),
        _ptr(temperature), _ptr(top_k), _ptr(seed), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
        _ptr(out.get("accept_prob")), _ptr(out.get("status")), sp))
    _check("spec_verify_static", code)
    return out


def verify_flat(target_rows: torch.Tensor, draft_rows: torch.Tensor, draft_tokens: torch.Tensor,
                lengths: torch.Tensor, temperature: Optional[torch.Tensor] = None,
                top_k: Optional[torch.Tensor] = None, seed: Optional[torch.Tensor] = None,
                out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_verify_flat on torch tensors: target_rows [sum(L+1), V], draft_rows [sum(L), V] hold only
    the verified rows, request after request; draft_tokens [B, gamma]; lengths [B] int32.  The row
    counts of the two tensors are passed on: a request whose rows lie past them gets REQ_BAD_ROWS."""
    lib = load_library()
    for name, t in (("target_rows", target_rows), ("draft_rows", draft_rows)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be [rows, V]")
    if not isinstance(draft_tokens, torch.Tensor) or draft_tokens.dim() != 2:
        raise ValueError("draft_tokens must be [B, gamma]")
    B, G = draft_tokens.shape
    V = target_rows.shape[1]
    if draft_rows.shape[1] != V:
        raise ValueError("draft_rows must be [sum(L), V] with the target rows' V")
    for name, t in (("lengths", lengths), ("temperature", temperature), ("top_k", top_k), ("seed", seed)):
        _vec(t, name, B)
    if lengths is None:
        raise ValueError("lengths are required (they define the layout)")
    _dev(target_rows, "target_rows", (torch.float32, torch.bfloat16), 2)
    _dev(draft_rows, "draft_rows", target_rows.dtype, 2)
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    _dev(lengths, "lengths", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    _dev(seed, "seed", _SEED_DTYPES, 1)
    dev = target_rows.device
    _on(dev, draft_rows=draft_rows, draft_tokens=draft_tokens, lengths=lengths, temperature=temperature,
        top_k=top_k, seed=seed)
    mine = []
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
        mine.append(temperature)
    if seed is None:
        seed = torch.zeros(B, dtype=torch.int64, device=dev)
        mine.append(seed)
    out = _verify_outputs(B, G, dev, out, mine)
    ws = _workspace(int(lib.spec_verify_workspace_size(B, G, V)), dev, workspace, mine)
    # an empty draft_rows tensor (every length 0) still needs an aligned non-null pointer
    n_drows = draft_rows.shape[0]
    drows = draft_rows
    if draft_rows.numel() == 0:
        drows = torch.empty((1, V), dtype=target_rows.dtype, device=dev)
        mine.append(drows)
    code = _launch(stream, mine, lambda sp: lib.spec_verify_flat(
        B, G, V, _logit_dtype(target_rows), _ptr(target_rows), target_rows.shape[0], _ptr(drows), n_drows,
        _ptr(draft_tokens), _ptr(lengths), _ptr(temperature), _ptr(top_k), _ptr(seed), _ptr(out["num_accepted"]),
        _ptr(out["out_tokens"]), _ptr(out.get("accept_prob")), _ptr(out.get("status")), _ptr(ws),
        ws.numel() * ws.element_size(), sp))
    _check("spec_verify_flat", code)
    return out


def verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, lengths: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_verify_greedy on torch tensors.  Returns dict(num_accepted, out_tokens, status)."""
    lib = load_library()
    if not isinstance(target, torch.Tensor) or target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    G = G1 - 1
    _shape(draft_tokens, "draft_tokens", (B, G))
    _vec(lengths, "lengths", B)
    _dev(target, "target", (torch.float32, torch.bfloat16), 3)
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    _dev(lengths, "lengths", torch.int32, 1)
    dev = target.device
    _on(dev, draft_tokens=draft_tokens, lengths=lengths)
    mine = []
    if out is None:
        out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(out.values())
    else:
        spec = _verify_out_spec(B, G)
        del spec["accept_prob"]
        _check_out(out, spec, dev)
    nbytes = int(lib.spec_verify_greedy_workspace_size(B, G))
    ws = _workspace(nbytes, dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_verify_greedy(
        B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft_tokens), _ptr(lengths), _ptr(out["num_accepted"]),
        _ptr(out["out_tokens"]), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_verify_greedy", code)
    return out


def _sched_inputs(conf, sps):
    if not isinstance(conf, torch.Tensor) or conf.dim() != 2:
        raise ValueError("conf must be [B, gamma]")
    if not isinstance(sps, torch.Tensor) or sps.dim() != 1:
        raise ValueError("sps must be a 1-D cost table")
    _dev(conf, "conf", torch.float32, 2)
    _dev(sps, "sps", torch.float64, 1)
    _on(conf.device, sps=sps)
    return conf.shape


def _sched_out_spec(B):
    return dict(lengths=((B,), torch.int32, True), theta=((1,), torch.float64, False),
                status=((B,), torch.int32, False))


def schedule_lengths(conf: torch.Tensor, sps: torch.Tensor, budget_tokens: int,
                     mode: int = SPEC_SCHED_EARLY_STOP, out: Optional[dict] = None, stream=None,
                     workspace: Optional[torch.Tensor] = None) -> dict:
    """spec_schedule_lengths on torch tensors.  Returns dict(lengths, theta, status)."""
    lib = load_library()
    B, G = _sched_inputs(conf, sps)
    dev = conf.device
    mine = []
    if out is None:
        out = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(out.values())
    else:
        _check_out(out, _sched_out_spec(B), dev)
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_schedule_lengths(
        B, G, _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens), int(mode), _ptr(out["lengths"]),
        _ptr(out.get("theta")), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_schedule_lengths", code)
    return out


def schedule_verify(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, conf: torch.Tensor,
                    sps: torch.Tensor, budget_tokens: int, mode: int = SPEC_SCHED_EARLY_STOP,
                    temperature: Optional[torch.Tensor] = None, top_k: Optional[torch.Tensor] = None,
                    seed: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                    workspace: Optional[torch.Tensor] = None, sched_workspace: Optional[torch.Tensor] = None,
                    stream=None, events=None, left_to_right: bool = False) -> dict:
    """spec_schedule_verify: the scheduler's lengths, then verification under the budget, in one call.

    Inputs as for schedule_lengths (conf, sps, budget_tokens, mode) and verify (no lengths).
    left_to_right: OR SPEC_VERIFY_LEFT_TO_RIGHT into the mode (the walk that stops at the first
    rejection; accept_prob NaN after it, rows after it not read).
    Returns dict(lengths, theta, sched_status, num_accepted, out_tokens, accept_prob, status).
    """
    lib = load_library()
    if isinstance(target, torch.Tensor) and target.dim() == 3:
        _shape(conf, "conf", (target.shape[0], target.shape[1] - 1))
    B, G, V, temperature, seed, mine = _verify_inputs(target, draft, draft_tokens, None, temperature, top_k, seed)
    _sched_inputs(conf, sps)
    dev = target.device
    _on(dev, conf=conf)
    if out is None:
        out = _verify_outputs(B, G, dev, None, mine)
        extra = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                     theta=torch.empty(1, dtype=torch.float64, device=dev),
                     sched_status=torch.empty(B, dtype=torch.int32, device=dev))
        out.update(extra)
        mine.extend(extra.values())
    else:
        spec = _verify_out_spec(B, G)
        spec.update(lengths=((B,), torch.int32, True), theta=((1,), torch.float64, False),
                    sched_status=((B,), torch.int32, False))
        _check_out(out, spec, dev)
    ws = _workspace(int(lib.spec_verify_workspace_size(B, G, V)), dev, workspace, mine)
    sws = _workspace(int(lib.spec_schedule_workspace_size(B, G)), dev, sched_workspace, mine)
    ev0, ev1 = _events(events)
    code = _launch(stream, mine, lambda sp: lib.spec_schedule_verify(
        B, G, V, _logit_dtype(target), _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens),
        int(mode) | (SPEC_VERIFY_LEFT_TO_RIGHT if left_to_right else 0),
        _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(temperature), _ptr(top_k), _ptr(seed),
        _ptr(out["lengths"]), _ptr(out.get("theta")), _ptr(out.get("sched_status")), _ptr(out["num_accepted"]),
        _ptr(out["out_tokens"]), _ptr(out.get("accept_prob")), _ptr(out.get("status")),
        _ptr(sws), sws.numel() * sws.element_size(), _ptr(ws), ws.numel() * ws.element_size(), sp, ev0, ev1))
    _check("spec_schedule_verify", code)
    return out


def overlap_mass(target: torch.Tensor, draft: torch.Tensor, lengths: Optional[torch.Tensor] = None,
                 temperature: Optional[torch.Tensor] = None, top_k: Optional[torch.Tensor] = None,
                 out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_overlap_mass on torch tensors.  Returns dict(overlap [B, gamma] float64, status [B])."""
    lib = load_library()
    if not isinstance(target, torch.Tensor) or target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    G = G1 - 1
    _shape(draft, "draft", (B, G, V))
    for name, t in (("lengths", lengths), ("temperature", temperature), ("top_k", top_k)):
        _vec(t, name, B)
    _dev(target, "target", (torch.float32, torch.bfloat16), 3)
    _dev(draft, "draft", target.dtype, 3)
    _dev(lengths, "lengths", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    dev = target.device
    _on(dev, draft=draft, lengths=lengths, temperature=temperature, top_k=top_k)
    mine = []
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
        mine.append(temperature)
    if out is None:
        out = dict(overlap=torch.empty((B, G), dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(out.values())
    else:
        _check_out(out, dict(overlap=((B, G), torch.float64, True), status=((B,), torch.int32, False)), dev)
    ws = _workspace(lib.spec_overlap_workspace_size(B, G, V), dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_overlap_mass(
        B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft), _ptr(lengths), _ptr(temperature), _ptr(top_k),
        _ptr(out["overlap"]), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_overlap_mass", code)
    return out


def draft_markov(base: torch.Tensor, W1: torch.Tensor, W2t: torch.Tensor, anchor: torch.Tensor,
                 temperature: Optional[torch.Tensor] = None, seed: Optional[torch.Tensor] = None,
                 hidden: Optional[torch.Tensor] = None, conf_w: Optional[torch.Tensor] = None,
                 out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                 in_place: bool = False, conf_tau: Optional[torch.Tensor] = None) -> dict:
    """spec_draft_markov on torch tensors.  Returns dict(tokens, logits, conf, status).

    base [B, gamma, V] (float32 or bfloat16); W1 and W2t [V, r] bfloat16 (W2t row v = column v of
    the r x V projection); anchor [B] int32; temperature [B] float32 (default ones); seed [B] int64
    (uint64 bit patterns, default zeros); hidden [B, gamma, d] (base's dtype) and conf_w [d + r]
    float32 for the confidences (conf_w alone when d = 0); conf_tau [gamma] float64 per-position
    temperatures of the confidences (sts_fit's output).  in_place writes the draft logits over
    `base`.
    """
    lib = load_library()
    if not isinstance(base, torch.Tensor) or base.dim() != 3:
        raise ValueError("base must be [B, gamma, V]")
    B, G, V = base.shape
    if not isinstance(W1, torch.Tensor) or W1.dim() != 2:
        raise ValueError("W1 must be [V, r]")
    r = W1.shape[1]
    _shape(W1, "W1", (V, r))
    _shape(W2t, "W2t", (V, r))
    for name, t in (("anchor", anchor), ("temperature", temperature), ("seed", seed)):
        _vec(t, name, B)
    d = 0
    if hidden is not None:
        if not isinstance(hidden, torch.Tensor) or hidden.dim() != 3 or tuple(hidden.shape[:2]) != (B, G):
            raise ValueError("hidden must be [B, gamma, d]")
        d = hidden.shape[2]
    if conf_w is not None:
        _vec(conf_w, "conf_w (d + r values)", d + r)
    _vec(conf_tau, "conf_tau (gamma values)", G)
    _dev(base, "base", (torch.float32, torch.bfloat16), 3)
    _dev(W1, "W1", torch.bfloat16, 2)
    _dev(W2t, "W2t", torch.bfloat16, 2)
    _dev(anchor, "anchor", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(seed, "seed", _SEED_DTYPES, 1)
    _dev(hidden, "hidden", base.dtype, 3)
    _dev(conf_w, "conf_w", torch.float32, 1)
    _dev(conf_tau, "conf_tau", torch.float64, 1)
    dev = base.device
    _on(dev, W1=W1, W2t=W2t, anchor=anchor, temperature=temperature, seed=seed, hidden=hidden, conf_w=conf_w,
        conf_tau=conf_tau)
    mine = []
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
        mine.append(temperature)
    if out is None:
        out = dict(tokens=torch.empty((B, G), dtype=torch.int32, device=dev),
                   logits=base if in_place else torch.empty_like(base),
                   conf=torch.empty((B, G), dtype=torch.float32, device=dev) if conf_w is not None else None,
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(t for k, t in out.items() if not (in_place and k == "logits"))
    else:
        _check_out(out, dict(tokens=((B, G), torch.int32, True), logits=((B, G, V), base.dtype, True),
                             conf=((B, G), torch.float32, False), status=((B,), torch.int32, True)), dev)
    nbytes = int(lib.spec_draft_workspace_size(B, G, V))
    ws = _workspace(nbytes, dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_draft_markov(
        B, G, V, r, _logit_dtype(base), _ptr(base), _ptr(W1), _ptr(W2t), _ptr(anchor), _ptr(temperature),
        _ptr(seed), d, _ptr(hidden), _ptr(conf_w), _ptr(conf_tau), _ptr(out["tokens"]), _ptr(out["logits"]),
        _ptr(out.get("conf")), _ptr(out["status"]), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_draft_markov", code)
    return out


def sts_fit(conf_logits: torch.Tensor, labels: torch.Tensor, taus: torch.Tensor, bins: int = 15,
            out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_sts_fit: conf_logits [N, gamma] float32, labels [N, gamma] uint8, taus [ntau] float64.
    Returns dict(tau [gamma] float64, index [gamma] int32, ece [gamma, ntau] float64)."""
    lib = load_library()
    if not isinstance(conf_logits, torch.Tensor) or conf_logits.dim() != 2:
        raise ValueError("conf_logits must be [N, gamma]")
    N, G = conf_logits.shape
    _shape(labels, "labels", (N, G))
    if not isinstance(taus, torch.Tensor) or taus.dim() != 1:
        raise ValueError("taus must be a 1-D grid")
    _dev(conf_logits, "conf_logits", torch.float32, 2)
    _dev(labels, "labels", torch.uint8, 2)
    _dev(taus, "taus", torch.float64, 1)
    ntau = taus.numel()
    dev = conf_logits.device
    _on(dev, labels=labels, taus=taus)
    mine = []
    if out is None:
        out = dict(tau=torch.empty(G, dtype=torch.float64, device=dev),
                   index=torch.empty(G, dtype=torch.int32, device=dev),
                   ece=torch.empty((G, ntau), dtype=torch.float64, device=dev))
        mine.extend(out.values())
    else:
        _check_out(out, dict(tau=((G,), torch.float64, True), index=((G,), torch.int32, False),
                             ece=((G, ntau), torch.float64, False)), dev)
    nbytes = int(lib.spec_sts_workspace_size(N, ntau, bins))
    ws = _workspace(nbytes, dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_sts_fit(
        N, G, _ptr(conf_logits), _ptr(labels), ntau, _ptr(taus), bins, _ptr(out["tau"]), _ptr(out.get("index")),
        _ptr(out.get("ece")), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_sts_fit", code)
    return out


def sts_apply(conf_logits: torch.Tensor, tau: torch.Tensor, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """spec_sts_apply: sigmoid(conf_logits / tau) per position, float32 [B, gamma]."""
    lib = load_library()
    if not isinstance(conf_logits, torch.Tensor) or conf_logits.dim() != 2:
        raise ValueError("conf_logits must be [B, gamma]")
    B, G = conf_logits.shape
    _vec(tau, "tau", G)
    _shape(out, "out", (B, G))
    _dev(conf_logits, "conf_logits", torch.float32, 2)
    _dev(tau, "tau", torch.float64, 1)
    _dev(out, "out", torch.float32, 2)
    _on(conf_logits.device, tau=tau, out=out)
    mine = []
    if out is None:
        out = torch.empty_like(conf_logits)
        mine.append(out)
    _check("spec_sts_apply", _launch(stream, mine, lambda sp: lib.spec_sts_apply(
        B, G, _ptr(conf_logits), _ptr(tau), _ptr(out), sp)))
    return out


def read_ceiling(data: torch.Tensor, nbytes: int, grid: int, sink: torch.Tensor, stream=None) -> None:
    """spec_read_ceiling: one plain read of the first `nbytes` of `data` (a measurement aid)."""
    lib = load_library()
    if not data.is_cuda or nbytes > data.numel() * data.element_size():
        raise ValueError("data must be a device tensor of at least nbytes")
    _check("spec_read_ceiling", lib.spec_read_ceiling(_ptr(data), int(nbytes), int(grid), _ptr(sink),
                                                      _stream(stream)))


def schedule_capacity(conf: torch.Tensor, sps: torch.Tensor, budget_tokens: int, out: Optional[dict] = None,
                      stream=None, workspace: Optional[torch.Tensor] = None) -> dict:
    """spec_schedule_capacity: dict(capacity [1] int32, theta [1] float64, status [B])."""
    lib = load_library()
    B, G = _sched_inputs(conf, sps)
    dev = conf.device
    mine = []
    if out is None:
        out = dict(capacity=torch.empty(1, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(out.values())
    else:
        _check_out(out, dict(capacity=((1,), torch.int32, True), theta=((1,), torch.float64, False),
                             status=((B,), torch.int32, False)), dev)
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_schedule_capacity(
        B, G, _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens), _ptr(out["capacity"]), _ptr(out.get("theta")),
        _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(), sp))
    _check("spec_schedule_capacity", code)
    return out


def schedule_topk(conf: torch.Tensor, capacity: torch.Tensor, out: Optional[dict] = None, stream=None,
                  workspace: Optional[torch.Tensor] = None) -> dict:
    """spec_schedule_topk: dict(lengths [B] int32, status [B]) admitting up to capacity[0] candidates."""
    lib = load_library()
    if not isinstance(conf, torch.Tensor) or conf.dim() != 2:
        raise ValueError("conf must be [B, gamma]")
    B, G = conf.shape
    _vec(capacity, "capacity", 1)
    _dev(conf, "conf", torch.float32, 2)
    _dev(capacity, "capacity", torch.int32, 1)
    dev = conf.device
    _on(dev, capacity=capacity)
    mine = []
    if out is None:
        out = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
        mine.extend(out.values())
    else:
        _check_out(out, dict(lengths=((B,), torch.int32, True), status=((B,), torch.int32, False)), dev)
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace, mine)
    code = _launch(stream, mine, lambda sp: lib.spec_schedule_topk(
        B, G, _ptr(conf), _ptr(capacity), _ptr(out["lengths"]), _ptr(out.get("status")), _ptr(ws),
        ws.numel() * ws.element_size(), sp))
    _check("spec_schedule_topk", code)
    return out


def philox_uniforms(seed: torch.Tensor, request: torch.Tensor, position: torch.Tensor, stream=None):
    """The library's (u_accept, u_emit) draws for each (seed, request, position) triple."""
    lib = load_library()
    n = seed.numel() if isinstance(seed, torch.Tensor) else -1
    for name, t in (("seed", seed), ("request", request), ("position", position)):
        _vec(t, name, n)
    _dev(seed, "seed", torch.int64, 1)
    _dev(request, "request", torch.int32, 1)
    _dev(position, "position", torch.int32, 1)
    _on(seed.device, request=request, position=position)
    ua = torch.empty(n, dtype=torch.float64, device=seed.device)
    ue = torch.empty(n, dtype=torch.float64, device=seed.device)
    code = _launch(stream, [ua, ue], lambda sp: lib.spec_philox_uniforms(
        n, _ptr(seed), _ptr(request), _ptr(position), _ptr(ua), _ptr(ue), sp))
    _check("spec_philox_uniforms", code)
    return ua, ue
