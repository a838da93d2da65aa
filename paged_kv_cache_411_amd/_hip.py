"""HIP events through the process's own HIP runtime (plumbing, like torch's
events, but with the creation flags torch does not expose).

An event recorded with the default flags releases to system scope (the L2
is written back and invalidated so that the host sees device memory); in the
middle of a stream of kernels that costs the next kernel several
microseconds. The decode step only needs an event to tell the host that the
kernels reading a pinned staging buffer have finished, and the benchmark only
needs kernel timestamps, so both use ``hipEventDisableSystemFence`` events.
"""

from __future__ import annotations

import ctypes
from typing import Optional

hipEventDisableTiming = 0x2
hipEventDisableSystemFence = 0x20000000

_rt: Optional[ctypes.CDLL] = None


def _loaded_runtime_path() -> str:
    """Path of the libamdhip64 this process has mapped (torch's, which the
    library shares), so that ctypes opens that one and not a second copy."""
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if line.strip() else ""
                if "/libamdhip64.so" in path:
                    return path
    except OSError:
        pass
    return "libamdhip64.so.7"


def runtime() -> ctypes.CDLL:
    """The HIP runtime already loaded in this process (torch's and the
    library's are one)."""
    global _rt
    if _rt is None:
        import torch  # noqa: F401  - loads the runtime
        r = ctypes.CDLL(_loaded_runtime_path())
        vp = ctypes.c_void_p
        r.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        r.hipEventRecord.argtypes = [vp, vp]
        r.hipEventQuery.argtypes = [vp]
        r.hipEventSynchronize.argtypes = [vp]
        r.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        r.hipEventDestroy.argtypes = [vp]
        for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventQuery", "hipEventSynchronize",
                  "hipEventElapsedTime", "hipEventDestroy"):
            getattr(r, f).restype = ctypes.c_int
        _rt = r
    return _rt


class Event:
    """A HIP event created with ``flags`` (default: timing on, no system-scope
    fence). ``handle`` is the hipEvent_t."""

    def __init__(self, timing: bool = True, system_fence: bool = False):
        r = runtime()
        flags = (0 if timing else hipEventDisableTiming) | (0 if system_fence else hipEventDisableSystemFence)
        h = ctypes.c_void_p()
        rc = r.hipEventCreateWithFlags(ctypes.byref(h), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = h.value
        self._r = r

    def record(self, stream: int) -> None:
        rc = self._r.hipEventRecord(self.handle, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def query(self) -> bool:
        """True once the work the event tracks has completed (or it was never recorded)."""
        rc = self._r.hipEventQuery(self.handle)
        if rc == 0:
            return True
        if rc == 600:   # hipErrorNotReady
            return False
        raise RuntimeError(f"hipEventQuery failed ({rc})")

    def synchronize(self) -> None:
        rc = self._r.hipEventSynchronize(self.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float()
        rc = self._r.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self._r.hipEventDestroy(h)
            self.handle = None
