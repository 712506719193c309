"""Helpers for the GPU parity tests: move seeded stored arrays to the device
and compare device results with the oracle."""
import numpy as np

from synth import to_dev, to_np  # noqa: F401  (re-exported for the tests)


def rel_err(x, y):
    """max |x - y| / max |y| over one tensor (y the oracle)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    assert np.all(np.isfinite(x)), "non-finite device output"
    den = np.max(np.abs(y)) if y.size else 0.0
    num = np.max(np.abs(x - y)) if y.size else 0.0
    return num / den if den > 0 else num


TOL = {"f32": 1e-4, "bf16": 2e-2}


class RawEvents:
    """hipEvent_t handles created through the process's HIP runtime (the one
    torch loaded), for the entry points' timing hooks; elapsed() fails unless
    both events were recorded."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = self.ct.c_void_p()
            assert self.hip.hipEventCreate(self.ct.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed(self, a, b):
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), self.ct.c_void_p(a), self.ct.c_void_p(b))
        assert rc == 0, "hipEventElapsedTime failed (%d): an event was not recorded" % rc
        return float(f.value)
