"""HIP events with explicit flags, through the HIP runtime that torch loaded.

torch.cuda.Event creates events whose record and wait carry system-scope
memory fences (a write-back of the L2 caches for the host's sake).  Events
that only order streams of one device, or time kernels, need none: the
kernels' own completion already makes their writes visible on the device.
This module creates such events (hipEventDisableSystemFence) and records and
waits on them; it is plumbing around the HIP runtime API, no computation.
"""
from __future__ import annotations

import ctypes as C
import os

HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Owns the hipEvent_t handles it creates; `close()` destroys them."""

    def __init__(self):
        import torch
        lib = C.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        lib.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        lib.hipEventDestroy.argtypes = [C.c_void_p]
        lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        lib.hipStreamWaitEvent.argtypes = [C.c_void_p, C.c_void_p, C.c_uint]
        self.lib = lib
        self.made = []

    def create(self, timing: bool = True) -> int:
        """A device-scope event (no system fence); timing-capable unless asked not."""
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else HIP_EVENT_DISABLE_TIMING)
        ev = C.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(C.byref(ev), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.made.append(ev.value)
        return ev.value

    def record(self, ev: int, stream) -> None:
        rc = self.lib.hipEventRecord(ev, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream, ev: int) -> None:
        """Work enqueued on `stream` after this call waits for `ev`."""
        rc = self.lib.hipStreamWaitEvent(stream.cuda_stream, ev, 0)
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def ms(self, a: int, b: int) -> float:
        out = C.c_float()
        rc = self.lib.hipEventElapsedTime(C.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self) -> None:
        for e in self.made:
            self.lib.hipEventDestroy(e)
        self.made = []
