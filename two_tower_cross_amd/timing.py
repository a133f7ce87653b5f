"""Timing events for measurements: hipEvent_t handles created with hipEventDisableSystemFence.

A default HIP event's record performs a system-scope release: it writes back and invalidates the
caches, leaves the GPU idle for several microseconds between the kernels it separates and makes the
next kernel start cold. Events that only measure time do not need that fence.
"""
from __future__ import annotations


class TimingEvent:
    """A hipEvent_t for timing only, created with hipEventDisableSystemFence: recording it does
    not write back and invalidate the caches (the default event's system-scope fence costs about
    5 us of idle GPU time per record and leaves the next kernel with cold caches). Same interface
    as the parts of torch.cuda.Event used here; the handle lives in the HIP runtime torch loaded."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            h = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self.cuda_event = None
        h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(h), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self):
        import torch
        rc = self.hip().hipEventRecord(self.cuda_event, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, other):
        """Milliseconds from this event to ``other`` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, other.cuda_event)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.cuda_event:
            self._hip.hipEventDestroy(self.cuda_event)
