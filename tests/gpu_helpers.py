"""Helpers for the GPU parity tests: move seeded stored arrays to the device
and compare device results with the oracle."""
import numpy as np


def to_dev(st, torch):
    """synth.Stored -> device tensor with identical stored bits."""
    if st is None:
        return None
    if st.dtype == "bf16":
        t = torch.from_numpy(st.raw.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(st.raw, dtype=np.float32))
    return t.to("cuda")


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


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
