"""hipEvent_t handles for timing individual launches, from the HIP runtime torch loaded."""

from __future__ import annotations

import ctypes
import os


def _runtime():
    import torch
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    return ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")


class EventSet:
    """n hipEvent_t handles (timing enabled) as a ctypes array for the C ABI."""

    def __init__(self, n: int):
        self.rt = _runtime()
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.rt.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.handles[i] = h
        self.n = n

    def synchronize(self):
        rc = self.rt.hipEventSynchronize(self.handles[self.n - 1])
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed: {rc}")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            if self.handles[i]:
                self.rt.hipEventDestroy(self.handles[i])
                self.handles[i] = None
