"""Raw HIP events (via the HIP runtime library) for timing a kernel launched inside libspecverify.

torch.cuda.Event objects cannot be recorded by foreign code, so the timing
events handed to spec_verify_profiled are created here with hipEventCreate.
"""

import ctypes

_hip = None


def _lib():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventCreate.restype = ctypes.c_int
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventDestroy.restype = ctypes.c_int
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.restype = ctypes.c_int
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.restype = ctypes.c_int
    return _hip


class HipEvent:
    """A HIP event; `.handle` is the hipEvent_t to pass as void*."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = _lib().hipEventCreate(ctypes.byref(h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.handle = h

    @property
    def cuda_event(self):
        return self.handle.value

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
