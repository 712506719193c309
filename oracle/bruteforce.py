"""Explicitly unrolled sums for tiny T -- a third implementation used only to
pin the recurrent oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Unrolling the per-slot gated RNN of "Gated Slot Attention for Efficient
Linear-Time Sequence Modeling" (Sec. 3.2) gives, for every slot c,
    Kt_t[c] = (prod_{i<=t} alpha_i[c]) Kt_0[c]
              + sum_{j<=t} (prod_{j<i<=t} alpha_i[c]) (1 - alpha_j[c]) k_j
and the same for Vt with v.  The gate alpha = sigmoid(g)^(1/tau) (Sec. 3.3) is
evaluated here directly in linear space (no logs), and every product is taken
with numpy.prod over the explicit token range.
"""
from __future__ import annotations

import numpy as np


def _alpha(g, tau):
    g = np.asarray(g, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-g))) ** (1.0 / tau)


def _read(z, nonlinearity):
    """Slot read weights from the slot scores: softmax (Sec. 3.2) or one of the
    element-wise ablations of Table 2, each written from its definition."""
    if nonlinearity == "softmax":
        e = np.exp(z - z.max())
        return e / e.sum()
    if nonlinearity == "identity":
        return z
    if nonlinearity == "swish":
        return z / (1.0 + np.exp(-z))
    if nonlinearity == "relu":
        return np.maximum(z, 0.0)
    if nonlinearity == "relu2":
        return np.maximum(z, 0.0) ** 2
    raise ValueError(nonlinearity)


def gsa_unit(q, k, v, g, k0=None, v0=None, tau=8.0, nonlinearity="softmax"):
    T, dk = q.shape
    m = g.shape[1]
    dv = v.shape[1]
    a = _alpha(g, tau)                      # [T, m]
    K0 = np.zeros((m, dk)) if k0 is None else np.asarray(k0, dtype=np.float64)
    V0 = np.zeros((m, dv)) if v0 is None else np.asarray(v0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        Kt = np.prod(a[: t + 1], axis=0)[:, None] * K0
        Vt = np.prod(a[: t + 1], axis=0)[:, None] * V0
        for j in range(t + 1):
            f = np.prod(a[j + 1: t + 1], axis=0) * (1.0 - a[j])     # [m]
            Kt = Kt + f[:, None] * k[j][None, :]
            Vt = Vt + f[:, None] * v[j][None, :]
        z = Kt @ q[t]
        o[t] = Vt.T @ _read(z, nonlinearity)
    return o


def gla_unit(q, k, v, g, s0=None, tau=16.0):
    T, dk = q.shape
    dv = v.shape[1]
    a = _alpha(g, tau)                      # [T, dk]
    S0 = np.zeros((dk, dv)) if s0 is None else np.asarray(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        St = np.prod(a[: t + 1], axis=0)[:, None] * S0
        for j in range(t + 1):
            f = np.prod(a[j + 1: t + 1], axis=0)                    # [dk]
            St = St + f[:, None] * np.outer(k[j], v[j])
        o[t] = St.T @ q[t]
    return o
