"""HIP events for the C ABI's optional kernel timer (muse_kernel_timer).

The events are created through the HIP runtime that torch has already loaded
in this process, so they can be recorded on torch's streams.
"""
from __future__ import annotations

import ctypes
import os

from . import KernelTimer

_hip = None


def hip() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name, mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
                break
            except OSError:
                continue
        if _hip is None:
            _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return _hip


class KernelTimers:
    """A pool of (start, stop) event pairs, one per timed call."""

    def __init__(self, n: int):
        h = hip()
        self.timers = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(a)) or h.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.timers.append(KernelTimer(a.value, b.value))

    def __getitem__(self, i: int) -> KernelTimer:
        return self.timers[i]

    def __len__(self) -> int:
        return len(self.timers)

    def elapsed_ms(self, i: int) -> float:
        t = self.timers[i]
        h = hip()
        if h.hipEventSynchronize(ctypes.c_void_p(t.stop)):
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(t.start), ctypes.c_void_p(t.stop)):
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        h = hip()
        for t in self.timers:
            h.hipEventDestroy(ctypes.c_void_p(t.start))
            h.hipEventDestroy(ctypes.c_void_p(t.stop))
        self.timers = []
