"""Raw HIP events (via the HIP runtime library) for timing a kernel launched inside libspecverify.

torch.cuda.Event objects cannot be recorded by foreign code, so the timing
events handed to spec_verify_profiled are created here with hipEventCreateWithFlags.
"""

import ctypes

_hip = None


def _lib():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventCreateWithFlags.restype = ctypes.c_int
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventDestroy.restype = ctypes.c_int
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.restype = ctypes.c_int
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.restype = ctypes.c_int
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventRecord.restype = ctypes.c_int
    return _hip


# Timing-only events: recording them skips the system-scope fence (cache write-back and
# invalidation) that would otherwise stall the stream around the timed kernel.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvent:
    """A HIP event; `.handle` is the hipEvent_t to pass as void*."""

    def __init__(self, flags: int = HIP_EVENT_DISABLE_SYSTEM_FENCE):
        h = ctypes.c_void_p()
        rc = _lib().hipEventCreateWithFlags(ctypes.byref(h), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = h

    @property
    def cuda_event(self):
        return self.handle.value

    def record(self, stream) -> None:
        """Record on a torch stream (or a raw hipStream_t as int / None for the null stream)."""
        h = getattr(stream, "cuda_stream", stream)
        rc = _lib().hipEventRecord(self.handle, ctypes.c_void_p(h) if h else None)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        _lib().hipEventSynchronize(end.handle)
        ms = ctypes.c_float()
        rc = _lib().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(self.handle)
        except Exception:
            pass
