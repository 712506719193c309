"""Pins for the oracle's slot read non-linearities (CPU only).

The ablation study of "Gated Slot Attention for Efficient Linear-Time Sequence
Modeling" (Sec. 4.1.3, Table 2) replaces the softmax that links the two passes
by no non-linearity, Swish, ReLU or ReLU^2, applied to each slot score.  The
recurrent C oracle's variants are pinned here against the independent numpy
chunk form and the unrolled sums (each with its own statement of the
functions), against closed forms (a fixed state read as two matrix products,
one slot as a first-order IIR filter from scipy), and against invariances that
single out each function (linearity, positive homogeneity of degree 1 and 2,
Swish tending to ReLU for large scores).
"""
import ctypes
import math

import numpy as np
import pytest
import scipy.signal
import scipy.special

from oracle import bruteforce, chunkwise

ELEMENTWISE = ["identity", "swish", "relu", "relu2"]
ALL = ["softmax"] + ELEMENTWISE


def _rand(B, H, T, dk, dv, m, init=True, seed=0, g_shift=0.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk)) / math.sqrt(dk)
    k = r.standard_normal((B, H, T, dk)) / math.sqrt(dk)
    v = r.standard_normal((B, H, T, dv)) / math.sqrt(dk)
    g = r.standard_normal((B, H, T, m)) + g_shift
    k0 = r.standard_normal((B, H, m, dk)) * 0.3 if init else None
    v0 = r.standard_normal((B, H, m, dv)) * 0.3 if init else None
    return q, k, v, g, k0, v0


def _rel(x, y):
    den = np.max(np.abs(y))
    return np.max(np.abs(x - y)) / (den if den > 0 else 1.0)


@pytest.mark.parametrize("nl", ALL)
@pytest.mark.parametrize("C", [1, 8, 64])
def test_recurrent_equals_chunkwise(oracle_mod, nl, C):
    for T in sorted({1, C, C + 1, 2 * C + 5}):
        q, k, v, g, k0, v0 = _rand(1, 2, T, 8, 6, 5, init=(T % 2 == 1), seed=3 * T + C)
        ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, nonlinearity=nl)
        o, kf, vf = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=C, nonlinearity=nl)
        assert _rel(ref["o"], o) < 1e-12, (nl, C, T)
        assert _rel(ref["kf"], kf) < 1e-12 and _rel(ref["vf"], vf) < 1e-12


@pytest.mark.parametrize("nl", ALL)
def test_bruteforce(oracle_mod, nl):
    q, k, v, g, k0, v0 = _rand(1, 1, 7, 5, 4, 6, seed=21)
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, nonlinearity=nl)
    ob = bruteforce.gsa_unit(q[0, 0], k[0, 0], v[0, 0], g[0, 0], k0[0, 0], v0[0, 0], tau=8.0,
                             nonlinearity=nl)
    assert _rel(ref["o"][0, 0], ob) < 1e-12


def test_softmax_code_is_the_method(oracle_mod):
    q, k, v, g, k0, v0 = _rand(2, 1, 30, 8, 8, 6, seed=5)
    a = oracle_mod.gsa_fwd(q, k, v, g, k0, v0)
    b = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nonlinearity="softmax")
    assert np.array_equal(a["o"], b["o"])


def test_scores_and_read_weights(oracle_mod):
    """The returned read weights are the function of the returned raw scores."""
    q, k, v, g, k0, v0 = _rand(1, 2, 40, 8, 8, 7, seed=6)
    fns = {"identity": lambda z: z, "swish": lambda z: z * scipy.special.expit(z),
           "relu": lambda z: np.clip(z, 0.0, None), "relu2": lambda z: np.square(np.clip(z, 0.0, None))}
    for nl, f in fns.items():
        ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, want_scores=True, nonlinearity=nl)
        assert _rel(ref["s"], f(ref["z"])) < 1e-15, nl
        # the raw scores do not depend on the read (pass 1 is unchanged)
        base = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, want_scores=True)
        assert np.array_equal(ref["z"], base["z"])
        assert np.array_equal(ref["kf"], base["kf"]) and np.array_equal(ref["vf"], base["vf"])


def test_identity_frozen_state_is_two_matmuls(oracle_mod):
    """alpha = 1 freezes both states at K0, V0; with no non-linearity the read
    is o_t = V0^T (K0 q_t), i.e. O = Q K0^T V0."""
    q, k, v, g, k0, v0 = _rand(2, 1, 17, 7, 5, 6, seed=9)
    g[:] = np.inf
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nonlinearity="identity")
    for b in range(2):
        assert _rel(ref["o"][b, 0], (q[b, 0] @ k0[b, 0].T) @ v0[b, 0]) < 1e-13


@pytest.mark.parametrize("nl", ELEMENTWISE)
def test_single_slot_closed_form(oracle_mod, nl):
    """m = 1: both slot rows are first-order IIR filters of k and v with pole
    alpha and gain 1 - alpha; the output is f(Kt_t . q_t) Vt_t."""
    r = np.random.default_rng(18)
    T, d = 50, 6
    q, k = r.standard_normal((2, 1, 1, T, d))
    v = r.standard_normal((1, 1, T, d))
    g = np.full((1, 1, T, 1), 0.3)
    alpha = scipy.special.expit(0.3) ** (1 / 8.0)
    K = scipy.signal.lfilter([1.0 - alpha], [1.0, -alpha], k[0, 0], axis=0)
    V = scipy.signal.lfilter([1.0 - alpha], [1.0, -alpha], v[0, 0], axis=0)
    z = np.sum(K * q[0, 0], axis=1)
    f = {"identity": z, "swish": z * scipy.special.expit(z), "relu": np.clip(z, 0.0, None),
         "relu2": np.clip(z, 0.0, None) ** 2}[nl]
    ref = oracle_mod.gsa_fwd(q, k, v, g, tau=8.0, nonlinearity=nl)
    assert _rel(ref["o"][0, 0], f[:, None] * V) < 1e-12


def test_homogeneity_in_q(oracle_mod):
    """The read is linear in q with no non-linearity, positively homogeneous
    of degree 1 under ReLU and of degree 2 under ReLU^2; none of these holds
    for the softmax."""
    q, k, v, g, k0, v0 = _rand(1, 2, 33, 8, 8, 5, seed=10)
    q2 = np.random.default_rng(1).standard_normal(q.shape) / 3
    o = lambda qq, nl: oracle_mod.gsa_fwd(qq, k, v, g, k0, v0, nonlinearity=nl)["o"]
    assert _rel(o(q + 2.0 * q2, "identity"), o(q, "identity") + 2.0 * o(q2, "identity")) < 1e-13
    assert _rel(o(3.0 * q, "relu"), 3.0 * o(q, "relu")) < 1e-14
    assert _rel(o(3.0 * q, "relu2"), 9.0 * o(q, "relu2")) < 1e-14
    assert _rel(o(-q, "identity"), -o(q, "identity")) < 1e-15
    assert _rel(o(3.0 * q, "softmax"), 3.0 * o(q, "softmax")) > 1e-3


def test_swish_tends_to_relu(oracle_mod):
    """Swish(c z) / c -> ReLU(z) as c grows (sigmoid(c z) -> step(z))."""
    q, k, v, g, k0, v0 = _rand(1, 1, 25, 8, 8, 6, seed=11)
    c = 1e6
    a = oracle_mod.gsa_fwd(c * q, k, v, g, k0, v0, nonlinearity="swish")["o"] / c
    b = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nonlinearity="relu")["o"]
    assert _rel(a, b) < 1e-12
    # and at small scores Swish is z/2 to first order: o(eps q) ~ eps o_identity(q) / 2
    eps = 1e-7
    a = oracle_mod.gsa_fwd(eps * q, k, v, g, k0, v0, nonlinearity="swish")["o"] / eps
    b = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nonlinearity="identity")["o"] / 2
    assert _rel(a, b) < 1e-6


@pytest.mark.parametrize("nl", ELEMENTWISE)
def test_decode_chain_equals_forward(oracle_mod, nl):
    q, k, v, g, k0, v0 = _rand(2, 2, 19, 8, 6, 5, seed=12)
    full = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nonlinearity=nl)
    ks, vs = k0.copy(), v0.copy()
    for t in range(19):
        o, ks, vs = oracle_mod.gsa_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t],
                                               ks, vs, nonlinearity=nl)
        assert _rel(o, full["o"][:, :, t]) < 1e-14
    assert _rel(ks, full["kf"]) < 1e-14 and _rel(vs, full["vf"]) < 1e-14


def test_bad_code_rejected(oracle_mod):
    q, k, v, g, k0, v0 = _rand(1, 1, 4, 4, 4, 4, seed=0)
    with pytest.raises(ValueError):
        oracle_mod.gsa_fwd(q, k, v, g, nonlinearity=7)
    with pytest.raises(KeyError):
        oracle_mod.gsa_fwd(q, k, v, g, nonlinearity="tanh")
    o = np.empty_like(v)
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    for bad in (-1, 5):
        assert oracle_mod._load().oracle_gsa_fwd_nl(p(q), p(k), p(v), p(g), None, None, p(o), None,
                                                    None, None, None, 1, 1, 4, 4, 4, 4, 8.0, bad,
                                                    1) == 1
