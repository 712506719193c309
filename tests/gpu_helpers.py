"""Helpers for the GPU parity tests: move seeded stored arrays to the device
and compare device results with the oracle."""
import numpy as np

import synth
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


# ---------------------------------------------- gate regimes (input edits)
# With alpha = sigmoid(g)^(1/8), the bf16 kernels run a 64-token chunk in the
# chunk form while every slot's decay over it stays >= 2^-90, with 16-token
# sub-chunk reference points while every slot's decay over each sub-chunk
# does, and as an exact token walk otherwise.

def gates_normal(x_mean, x_std):
    """Gate logits N(x_mean, x_std) on every slot of every token (a decay
    regime chosen relative to the factorised forms' floor of 2^-90)."""
    def mut(inp):
        r = np.random.default_rng(5)
        inp["g"] = synth.stored(x_mean + x_std * r.standard_normal(inp["g"].shape), inp["g"].dtype)
    return mut


def gates_fast_slots(n, mean, std=1.0, seed=6):
    """Gate logits N(mean, std) on the first n slots of every token (a few
    slots forgetting fast), the stored N(0, 1) logits elsewhere."""
    def mut(inp):
        x = inp["g"].f64.copy()
        r = np.random.default_rng(seed)
        x[..., :n] = mean + std * r.standard_normal(x[..., :n].shape)
        inp["g"] = synth.stored(x, inp["g"].dtype)
    return mut


def gates_regime_per_chunk(inp):
    """One decay regime per 64-token chunk: 0 plain (chunk form); 1 g = -12 on
    every slot (64-token products ~2^-138, 16-token ~2^-35: sub-chunk form);
    2 g = -inf on one slot for three tokens (a 16-token product below 2^-90:
    exact walk); 3 g ~ N(-10, 1) on 8 slots (sub-chunk form); 4 g = -30.5 on
    4 slots (16-token products ~2^-88, the sub-chunk form near its floor);
    the ragged tail plain."""
    x = inp["g"].f64.copy()
    m = x.shape[-1]
    x[..., 64:128, :] = -12.0
    x[..., 130:133, m // 2] = -np.inf
    r = np.random.default_rng(8)
    x[..., 192:256, :8] = -10.0 + r.standard_normal(x[..., 192:256, :8].shape)
    x[..., 256:320, m - 4:] = -30.5
    inp["g"] = synth.stored(x, inp["g"].dtype)


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
