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

REQ_BAD_TOKEN = 1
REQ_BAD_TEMPERATURE = 2
REQ_NONFINITE = 4
REQ_BAD_LENGTH = 8
REQ_BAD_TOPK = 16
REQ_BAD_CONFIDENCE = 32

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
    "spec_verify_flat": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_verify_greedy_workspace_size": (_Z, [_I, _I]),
    "spec_verify_greedy": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_schedule_workspace_size": (_Z, [_I, _I]),
    "spec_schedule_lengths": (_I, [_I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "spec_schedule_verify": (_I, [_I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _Z, _P, _Z, _P, _P, _P]),
    "spec_philox_uniforms": (_I, [_I, _P, _P, _P, _P, _P, _P]),
    "spec_read_ceiling": (_I, [_P, _Z, _I, _P, _P]),
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


def _logit_dtype(t):
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def verify_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return int(load_library().spec_verify_workspace_size(B, gamma, V))


def _workspace(nbytes: int, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _verify_inputs(target, draft, draft_tokens, lengths, temperature, top_k, seed):
    """Checks the verify inputs; returns (B, gamma, V, temperature, seed) with the defaults filled in."""
    _dev(target, "target", (torch.float32, torch.bfloat16), 3)
    _dev(draft, "draft", target.dtype, 3)
    B, G1, V = target.shape
    G = G1 - 1
    if tuple(draft.shape) != (B, G, V):
        raise ValueError("draft must be [B, gamma, V]")
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    if tuple(draft_tokens.shape) != (B, G):
        raise ValueError("draft_tokens must be [B, gamma]")
    dev = target.device
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
    if seed is None:
        seed = torch.zeros(B, dtype=torch.int64, device=dev)
    _dev(lengths, "lengths", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    _dev(seed, "seed", (torch.int64, torch.uint64) if hasattr(torch, "uint64") else torch.int64, 1)
    return B, G, V, temperature, seed


def _verify_outputs(B, G, dev, out):
    """A caller's `out` is used as given (a missing accept_prob or status is passed as NULL)."""
    if out is None:
        out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, G + 1), dtype=torch.int32, device=dev),
                   accept_prob=torch.empty((B, G), dtype=torch.float32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
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
    """
    lib = load_library()
    B, G, V, temperature, seed = _verify_inputs(target, draft, draft_tokens, lengths, temperature, top_k, seed)
    dev = target.device
    out = _verify_outputs(B, G, dev, out)
    nbytes = int(lib.spec_verify_workspace_size(B, G, V))
    ws = _workspace(nbytes, dev, workspace)
    ev0, ev1 = _events(events)
    args = (B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(lengths),
            _ptr(temperature), _ptr(top_k), _ptr(seed), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
            _ptr(out.get("accept_prob")), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(),
            _stream(stream))
    if max_tokens is None:
        code = lib.spec_verify_profiled(*args, ev0, ev1)
    else:
        code = lib.spec_verify_bounded(*args, int(max_tokens), ev0, ev1)
    _check("spec_verify", code)
    return out


def verify_flat(target_rows: torch.Tensor, draft_rows: torch.Tensor, draft_tokens: torch.Tensor,
                lengths: torch.Tensor, temperature: Optional[torch.Tensor] = None,
                top_k: Optional[torch.Tensor] = None, seed: Optional[torch.Tensor] = None,
                out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_verify_flat on torch tensors: target_rows [sum(L+1), V], draft_rows [sum(L), V] hold only
    the verified rows, request after request; draft_tokens [B, gamma]; lengths [B] int32."""
    lib = load_library()
    _dev(target_rows, "target_rows", (torch.float32, torch.bfloat16), 2)
    _dev(draft_rows, "draft_rows", target_rows.dtype, 2)
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    _dev(lengths, "lengths", torch.int32, 1)
    B, G = draft_tokens.shape
    V = target_rows.shape[1]
    if draft_rows.shape[1] != V or lengths.numel() != B:
        raise ValueError("draft_rows must be [sum(L), V] and lengths [B]")
    dev = target_rows.device
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
    if seed is None:
        seed = torch.zeros(B, dtype=torch.int64, device=dev)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    _dev(seed, "seed", (torch.int64, torch.uint64) if hasattr(torch, "uint64") else torch.int64, 1)
    if out is None:
        out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, G + 1), dtype=torch.int32, device=dev),
                   accept_prob=torch.empty((B, G), dtype=torch.float32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(int(lib.spec_verify_workspace_size(B, G, V)), dev, workspace)
    # an empty draft_rows tensor (every length 0) still needs an aligned non-null pointer
    drows = draft_rows if draft_rows.numel() else torch.empty((1, V), dtype=target_rows.dtype, device=dev)
    code = lib.spec_verify_flat(
        B, G, V, _logit_dtype(target_rows), _ptr(target_rows), _ptr(drows), _ptr(draft_tokens), _ptr(lengths),
        _ptr(temperature), _ptr(top_k), _ptr(seed), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
        _ptr(out.get("accept_prob")), _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream))
    _check("spec_verify_flat", code)
    return out


def verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, lengths: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_verify_greedy on torch tensors.  Returns dict(num_accepted, out_tokens, status)."""
    lib = load_library()
    _dev(target, "target", (torch.float32, torch.bfloat16), 3)
    B, G1, V = target.shape
    G = G1 - 1
    _dev(draft_tokens, "draft_tokens", torch.int32, 2)
    if tuple(draft_tokens.shape) != (B, G):
        raise ValueError("draft_tokens must be [B, gamma]")
    _dev(lengths, "lengths", torch.int32, 1)
    dev = target.device
    if out is None:
        out = dict(num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    nbytes = int(lib.spec_verify_greedy_workspace_size(B, G))
    ws = _workspace(nbytes, dev, workspace)
    code = lib.spec_verify_greedy(B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft_tokens),
                                  _ptr(lengths), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
                                  _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("spec_verify_greedy", code)
    return out


def schedule_lengths(conf: torch.Tensor, sps: torch.Tensor, budget_tokens: int,
                     mode: int = SPEC_SCHED_EARLY_STOP, out: Optional[dict] = None, stream=None,
                     workspace: Optional[torch.Tensor] = None) -> dict:
    """spec_schedule_lengths on torch tensors.  Returns dict(lengths, theta, status)."""
    lib = load_library()
    _dev(conf, "conf", torch.float32, 2)
    _dev(sps, "sps", torch.float64, 1)
    B, G = conf.shape
    dev = conf.device
    if out is None:
        out = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace)
    code = lib.spec_schedule_lengths(B, G, _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens), int(mode),
                                     _ptr(out["lengths"]), _ptr(out.get("theta")), _ptr(out.get("status")),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("spec_schedule_lengths", code)
    return out


def schedule_verify(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, conf: torch.Tensor,
                    sps: torch.Tensor, budget_tokens: int, mode: int = SPEC_SCHED_EARLY_STOP,
                    temperature: Optional[torch.Tensor] = None, top_k: Optional[torch.Tensor] = None,
                    seed: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                    workspace: Optional[torch.Tensor] = None, sched_workspace: Optional[torch.Tensor] = None,
                    stream=None, events=None) -> dict:
    """spec_schedule_verify: the scheduler's lengths, then verification under the budget, in one call.

    Inputs as for schedule_lengths (conf, sps, budget_tokens, mode) and verify (no lengths).
    Returns dict(lengths, theta, sched_status, num_accepted, out_tokens, accept_prob, status).
    """
    lib = load_library()
    B, G, V, temperature, seed = _verify_inputs(target, draft, draft_tokens, None, temperature, top_k, seed)
    _dev(conf, "conf", torch.float32, 2)
    _dev(sps, "sps", torch.float64, 1)
    if tuple(conf.shape) != (B, G):
        raise ValueError("conf must be [B, gamma]")
    dev = target.device
    if out is None:
        out = _verify_outputs(B, G, dev, None)
        out.update(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   sched_status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(int(lib.spec_verify_workspace_size(B, G, V)), dev, workspace)
    sws = _workspace(int(lib.spec_schedule_workspace_size(B, G)), dev, sched_workspace)
    ev0, ev1 = _events(events)
    code = lib.spec_schedule_verify(
        B, G, V, _logit_dtype(target), _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens), int(mode),
        _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(temperature), _ptr(top_k), _ptr(seed),
        _ptr(out["lengths"]), _ptr(out.get("theta")), _ptr(out.get("sched_status")), _ptr(out["num_accepted"]),
        _ptr(out["out_tokens"]), _ptr(out.get("accept_prob")), _ptr(out.get("status")),
        _ptr(sws), sws.numel() * sws.element_size(), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
        ev0, ev1)
    _check("spec_schedule_verify", code)
    return out


def overlap_mass(target: torch.Tensor, draft: torch.Tensor, lengths: Optional[torch.Tensor] = None,
                 temperature: Optional[torch.Tensor] = None, top_k: Optional[torch.Tensor] = None,
                 out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_overlap_mass on torch tensors.  Returns dict(overlap [B, gamma] float64, status [B])."""
    lib = load_library()
    B, G1, V = target.shape
    G = G1 - 1
    _dev(target, "target", None, 3)
    _dev(draft, "draft", target.dtype, 3)
    _dev(lengths, "lengths", torch.int32, 1)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(top_k, "top_k", torch.int32, 1)
    if tuple(draft.shape) != (B, G, V):
        raise ValueError("draft must be [B, gamma, V] with target [B, gamma+1, V]")
    dev = target.device
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
    if out is None:
        out = dict(overlap=torch.empty((B, G), dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(lib.spec_overlap_workspace_size(B, G, V), dev, workspace)
    code = lib.spec_overlap_mass(B, G, V, _logit_dtype(target), _ptr(target), _ptr(draft), _ptr(lengths),
                                 _ptr(temperature), _ptr(top_k), _ptr(out["overlap"]), _ptr(out.get("status")),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
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
    _dev(base, "base", (torch.float32, torch.bfloat16), 3)
    B, G, V = base.shape
    _dev(W1, "W1", torch.bfloat16, 2)
    _dev(W2t, "W2t", torch.bfloat16, 2)
    r = W1.shape[1]
    if tuple(W1.shape) != (V, r) or tuple(W2t.shape) != (V, r):
        raise ValueError("W1 and W2t must be [V, r]")
    _dev(anchor, "anchor", torch.int32, 1)
    dev = base.device
    if temperature is None:
        temperature = torch.ones(B, dtype=torch.float32, device=dev)
    _dev(temperature, "temperature", torch.float32, 1)
    _dev(seed, "seed", (torch.int64, torch.uint64) if hasattr(torch, "uint64") else torch.int64, 1)
    d = 0
    if hidden is not None:
        _dev(hidden, "hidden", base.dtype, 3)
        if tuple(hidden.shape[:2]) != (B, G):
            raise ValueError("hidden must be [B, gamma, d]")
        d = hidden.shape[2]
    if conf_w is not None:
        _dev(conf_w, "conf_w", torch.float32, 1)
        if conf_w.numel() != d + r:
            raise ValueError("conf_w must hold d + r values")
    if conf_tau is not None:
        _dev(conf_tau, "conf_tau", torch.float64, 1)
        if conf_tau.numel() != G:
            raise ValueError("conf_tau must hold gamma values")
    if out is None:
        out = dict(tokens=torch.empty((B, G), dtype=torch.int32, device=dev),
                   logits=base if in_place else torch.empty_like(base),
                   conf=torch.empty((B, G), dtype=torch.float32, device=dev) if conf_w is not None else None,
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    nbytes = int(lib.spec_draft_workspace_size(B, G, V))
    ws = _workspace(nbytes, dev, workspace)
    code = lib.spec_draft_markov(B, G, V, r, _logit_dtype(base), _ptr(base), _ptr(W1), _ptr(W2t), _ptr(anchor),
                                 _ptr(temperature), _ptr(seed), d, _ptr(hidden), _ptr(conf_w), _ptr(conf_tau),
                                 _ptr(out["tokens"]),
                                 _ptr(out["logits"]), _ptr(out.get("conf")), _ptr(out["status"]), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check("spec_draft_markov", code)
    return out


def sts_fit(conf_logits: torch.Tensor, labels: torch.Tensor, taus: torch.Tensor, bins: int = 15,
            out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """spec_sts_fit: conf_logits [N, gamma] float32, labels [N, gamma] uint8, taus [ntau] float64.
    Returns dict(tau [gamma] float64, index [gamma] int32, ece [gamma, ntau] float64)."""
    lib = load_library()
    _dev(conf_logits, "conf_logits", torch.float32, 2)
    _dev(labels, "labels", torch.uint8, 2)
    _dev(taus, "taus", torch.float64, 1)
    N, G = conf_logits.shape
    if tuple(labels.shape) != (N, G):
        raise ValueError("labels must be [N, gamma]")
    ntau = taus.numel()
    dev = conf_logits.device
    if out is None:
        out = dict(tau=torch.empty(G, dtype=torch.float64, device=dev),
                   index=torch.empty(G, dtype=torch.int32, device=dev),
                   ece=torch.empty((G, ntau), dtype=torch.float64, device=dev))
    nbytes = int(lib.spec_sts_workspace_size(N, ntau, bins))
    ws = _workspace(nbytes, dev, workspace)
    code = lib.spec_sts_fit(N, G, _ptr(conf_logits), _ptr(labels), ntau, _ptr(taus), bins, _ptr(out["tau"]),
                            _ptr(out.get("index")), _ptr(out.get("ece")), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    _check("spec_sts_fit", code)
    return out


def sts_apply(conf_logits: torch.Tensor, tau: torch.Tensor, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """spec_sts_apply: sigmoid(conf_logits / tau) per position, float32 [B, gamma]."""
    lib = load_library()
    _dev(conf_logits, "conf_logits", torch.float32, 2)
    _dev(tau, "tau", torch.float64, 1)
    B, G = conf_logits.shape
    if out is None:
        out = torch.empty_like(conf_logits)
    _check("spec_sts_apply", lib.spec_sts_apply(B, G, _ptr(conf_logits), _ptr(tau), _ptr(out), _stream(stream)))
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
    _dev(conf, "conf", torch.float32, 2)
    _dev(sps, "sps", torch.float64, 1)
    B, G = conf.shape
    dev = conf.device
    if out is None:
        out = dict(capacity=torch.empty(1, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace)
    code = lib.spec_schedule_capacity(B, G, _ptr(conf), _ptr(sps), sps.numel(), int(budget_tokens),
                                      _ptr(out["capacity"]), _ptr(out.get("theta")), _ptr(out.get("status")),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("spec_schedule_capacity", code)
    return out


def schedule_topk(conf: torch.Tensor, capacity: torch.Tensor, out: Optional[dict] = None, stream=None,
                  workspace: Optional[torch.Tensor] = None) -> dict:
    """spec_schedule_topk: dict(lengths [B] int32, status [B]) admitting up to capacity[0] candidates."""
    lib = load_library()
    _dev(conf, "conf", torch.float32, 2)
    _dev(capacity, "capacity", torch.int32, 1)
    B, G = conf.shape
    dev = conf.device
    if out is None:
        out = dict(lengths=torch.empty(B, dtype=torch.int32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    ws = _workspace(lib.spec_schedule_workspace_size(B, G), dev, workspace)
    code = lib.spec_schedule_topk(B, G, _ptr(conf), _ptr(capacity), _ptr(out["lengths"]), _ptr(out.get("status")),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("spec_schedule_topk", code)
    return out


def philox_uniforms(seed: torch.Tensor, request: torch.Tensor, position: torch.Tensor, stream=None):
    """The library's (u_accept, u_emit) draws for each (seed, request, position) triple."""
    lib = load_library()
    _dev(seed, "seed", torch.int64, 1)
    _dev(request, "request", torch.int32, 1)
    _dev(position, "position", torch.int32, 1)
    n = seed.numel()
    ua = torch.empty(n, dtype=torch.float64, device=seed.device)
    ue = torch.empty(n, dtype=torch.float64, device=seed.device)
    code = lib.spec_philox_uniforms(n, _ptr(seed), _ptr(request), _ptr(position), _ptr(ua), _ptr(ue),
                                    _stream(stream))
    _check("spec_philox_uniforms", code)
    return ua, ue
