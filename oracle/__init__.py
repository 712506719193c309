"""CPU oracle for Gated Slot Attention and gated linear attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check in
``__graft_entry__`` and by the benchmark's CPU-baseline leg, never by the
product package.  It shares no code with the HIP path.

Three independent implementations, all float64:

* ``gsa_fwd`` / ``gla_fwd`` / ``gsa_decode_step`` -- the plain token-by-token
  recurrences, in C (``gsa_oracle.c``), the reference everything is measured
  against; ``gsa_bwd``, the gradients of ``gsa_fwd`` by reverse-mode
  differentiation of that recurrence (pinned by central differences of the
  forward);
* ``chunkwise`` -- the chunk decomposition of the paper's App. A.1 / App. B,
  written in numpy, used only to pin the recurrence;
* ``bruteforce`` -- explicitly unrolled sums for tiny T, likewise a pin.

Source: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
(arXiv 2409.07146), Sec. 2.3, Sec. 3.2-3.3, App. A-B.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (plain -O2, OpenMP over independent units)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L = ctypes.c_long
        D = ctypes.c_double
        I = ctypes.c_int
        lib.oracle_gsa_fwd.argtypes = [P] * 11 + [L] * 6 + [D, I]
        lib.oracle_gla_fwd.argtypes = [P] * 7 + [L] * 5 + [D, I]
        lib.oracle_gsa_decode_step.argtypes = [P] * 7 + [L] * 5 + [D, I]
        lib.oracle_gsa_fwd_nl.argtypes = [P] * 11 + [L] * 6 + [D, I, I]
        lib.oracle_gla_fwd_gm.argtypes = [P] * 7 + [L] * 5 + [D, I, I]
        lib.oracle_gsa_decode_step_nl.argtypes = [P] * 7 + [L] * 5 + [D, I, I]
        lib.oracle_gsa_bwd.argtypes = [P] * 15 + [L] * 6 + [D, I]
        lib.oracle_gsa_bwd_nl.argtypes = [P] * 15 + [L] * 6 + [D, I, I]
        for f in (lib.oracle_gsa_fwd, lib.oracle_gla_fwd, lib.oracle_gsa_decode_step,
                  lib.oracle_gsa_fwd_nl, lib.oracle_gsa_decode_step_nl, lib.oracle_gla_fwd_gm,
                  lib.oracle_gsa_bwd, lib.oracle_gsa_bwd_nl):
            f.restype = I
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


# Slot read non-linearity: the softmax over the slots (Sec. 3.2) or one of the
# element-wise replacements of the ablation study (Table 2).
NONLINEARITIES = {"softmax": 0, "identity": 1, "swish": 2, "relu": 3, "relu2": 4}


def _nl(nonlinearity) -> int:
    if isinstance(nonlinearity, str):
        return NONLINEARITIES[nonlinearity]
    if int(nonlinearity) not in NONLINEARITIES.values():
        raise ValueError("unknown slot non-linearity %r" % (nonlinearity,))
    return int(nonlinearity)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gsa_fwd(q, k, v, g, k0=None, v0=None, tau=8.0, want_states=True,
            want_scores=False, nthreads=1, nonlinearity="softmax"):
    """Recurrent GSA forward.  q,k [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T,m];
    k0 [B,H,m,dk], v0 [B,H,m,dv] optional.  Returns dict with o, and the final
    states kf/vf, slot read weights s (the softmax unless another
    nonlinearity is named) and raw slot scores z when asked for."""
    q, k, v, g, k0, v0 = map(_f64, (q, k, v, g, k0, v0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    m = g.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and g.shape[:3] == (B, H, T)
    if k0 is not None:
        assert k0.shape == (B, H, m, dk)
    if v0 is not None:
        assert v0.shape == (B, H, m, dv)
    o = np.empty((B, H, T, dv))
    kf = np.empty((B, H, m, dk)) if want_states else None
    vf = np.empty((B, H, m, dv)) if want_states else None
    s = np.empty((B, H, T, m)) if want_scores else None
    z = np.empty((B, H, T, m)) if want_scores else None
    rc = _load().oracle_gsa_fwd_nl(_p(q), _p(k), _p(v), _p(g), _p(k0), _p(v0), _p(o), _p(kf),
                                   _p(vf), _p(s), _p(z), B, H, T, dk, dv, m, float(tau),
                                   _nl(nonlinearity), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gsa_fwd failed (%d)" % rc)
    return dict(o=o, kf=kf, vf=vf, s=s, z=z)


def gsa_bwd(q, k, v, g, do, k0=None, v0=None, dkf=None, dvf=None, tau=8.0, nthreads=1,
            nonlinearity="softmax"):
    """Gradients of the recurrent GSA forward (with the slot read named by
    nonlinearity, as for gsa_fwd) by reverse-mode
    differentiation of the token recurrence.  do [B,H,T,dv] is the gradient of
    the outputs; dkf [B,H,m,dk] / dvf [B,H,m,dv] (optional) those of the final
    states.  Returns dict with dq, dk, dv, dg (shaped like q, k, v, g) and
    dk0 / dv0, the gradients of the initial states (zero states when k0 / v0
    are not given)."""
    q, k, v, g, do, k0, v0, dkf, dvf = map(_f64, (q, k, v, g, do, k0, v0, dkf, dvf))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    m = g.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and g.shape[:3] == (B, H, T)
    assert do.shape == v.shape
    for x, d in ((k0, dk), (dkf, dk), (v0, dv), (dvf, dv)):
        if x is not None:
            assert x.shape == (B, H, m, d)
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v), dg=np.empty_like(g),
               dk0=np.empty((B, H, m, dk)), dv0=np.empty((B, H, m, dv)))
    rc = _load().oracle_gsa_bwd_nl(_p(q), _p(k), _p(v), _p(g), _p(do), _p(k0), _p(v0), _p(dkf),
                                   _p(dvf), *(_p(out[n]) for n in ("dq", "dk", "dv", "dg", "dk0", "dv0")),
                                   B, H, T, dk, dv, m, float(tau), _nl(nonlinearity), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gsa_bwd failed (%d)" % rc)
    return out


GATE_INPUTS = {"logit": 0, "log_decay": 1}


def gla_fwd(q, k, v, g, s0=None, tau=16.0, want_state=True, nthreads=1, gate="logit"):
    """Recurrent GLA forward.  q,k,g [B,H,T,dk]; v [B,H,T,dv]; s0 [B,H,dk,dv].
    gate: "logit" (alpha = sigmoid(g)^(1/tau)) or "log_decay" (alpha =
    exp(min(g, 0)), tau unused)."""
    q, k, v, g, s0 = map(_f64, (q, k, v, g, s0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, H, T)
    o = np.empty((B, H, T, dv))
    sf = np.empty((B, H, dk, dv)) if want_state else None
    rc = _load().oracle_gla_fwd_gm(_p(q), _p(k), _p(v), _p(g), _p(s0), _p(o), _p(sf),
                                   B, H, T, dk, dv, float(tau), GATE_INPUTS[gate], int(nthreads))
    if rc:
        raise RuntimeError("oracle_gla_fwd failed (%d)" % rc)
    return dict(o=o, sf=sf)


def gsa_decode_step(q, k, v, g, kstate, vstate, tau=8.0, nthreads=1, nonlinearity="softmax"):
    """One recurrent GSA step.  q,k [N,H,dk]; v [N,H,dv]; g [N,H,m];
    kstate [N,H,m,dk], vstate [N,H,m,dv].  Returns (o, new_kstate, new_vstate);
    the inputs are not modified."""
    q, k, v, g = map(_f64, (q, k, v, g))
    ks = np.array(kstate, dtype=np.float64, copy=True, order="C")
    vs = np.array(vstate, dtype=np.float64, copy=True, order="C")
    N, H, dk = q.shape
    dv = v.shape[-1]
    m = g.shape[-1]
    assert ks.shape == (N, H, m, dk) and vs.shape == (N, H, m, dv)
    o = np.empty((N, H, dv))
    rc = _load().oracle_gsa_decode_step_nl(_p(q), _p(k), _p(v), _p(g), _p(ks), _p(vs), _p(o),
                                           N, H, dk, dv, m, float(tau), _nl(nonlinearity),
                                           int(nthreads))
    if rc:
        raise RuntimeError("oracle_gsa_decode_step failed (%d)" % rc)
    return o, ks, vs
