"""Device-memory plumbing for the layer: torch allocations of the packed weights and
activations, and the C-ABI weight descriptors pointing into them.  No arithmetic."""
from __future__ import annotations

import numpy as np

from . import _lib

_SIGNED = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}


def to_device(arr, device="cuda"):
    """Copy a numpy array to the device bit for bit (unsigned types travel as signed views)."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype in _SIGNED:
        a = a.view(_SIGNED[a.dtype])
    return torch.from_numpy(a).to(device)


def to_host(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


class LayerWeights:
    """One weight set on the device: E routed experts (groups 0..E-1) and the shared expert
    (group E) in the packed int4-g64 format."""

    KEYS = ("gate_up_q", "gate_up_s", "gate_up_b", "down_q", "down_s", "down_b")

    def __init__(self, w: dict, E: int, device="cuda"):
        self.E = E
        self.t = {key: to_device(w[key], device) for key in self.KEYS}

    def _ffn(self, g):
        t = self.t
        return _lib.q4_ffn(
            _lib.q4(t["gate_up_q"][g].data_ptr(), t["gate_up_s"][g].data_ptr(), t["gate_up_b"][g].data_ptr()),
            _lib.q4(t["down_q"][g].data_ptr(), t["down_s"][g].data_ptr(), t["down_b"][g].data_ptr()))

    @property
    def experts(self):
        return self._ffn(0)

    @property
    def shared(self):
        return self._ffn(self.E)

    def nbytes(self):
        return sum(v.numel() * v.element_size() for v in self.t.values())


def workspace(shp, device="cuda"):
    import torch
    n = _lib.moe_workspace_bytes(shp)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


# ---- HIP timing events (raw handles), created without the system-scope fence that a default
# event performs when it completes (a cache write-back and invalidate that slows the work after
# it): these events only time.
_HIP = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def _hip():
    """The HIP runtime that torch has already loaded."""
    global _HIP
    if _HIP is None:
        import ctypes
        _HIP = ctypes.CDLL("libamdhip64.so")
    return _HIP


def hip_event() -> int:
    """A timing HIP event without the system-scope fence on completion (raw handle)."""
    import ctypes
    e = ctypes.c_void_p()
    rc = _hip().hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE))
    if rc != 0:
        raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
    return e.value


def hip_event_record(e: int, stream) -> None:
    import ctypes
    rc = _hip().hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"hipEventRecord failed ({rc})")


def hip_elapsed_ms(a: int, b: int) -> float:
    import ctypes
    ms = ctypes.c_float()
    rc = _hip().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return ms.value


def hip_event_destroy(e: int) -> None:
    import ctypes
    _hip().hipEventDestroy(ctypes.c_void_p(e))
