"""Pins for the float64 oracle (CPU only).

The oracle is the plain recurrence of "Gated Slot Attention for Efficient
Linear-Time Sequence Modeling" (Sec. 3.2-3.3).  It is pinned here against
things other than itself: the independent chunkwise implementation (App. A.1
/ App. B), explicitly unrolled sums, closed forms that reduce to textbook or
library routines (linear attention as a masked matmul, a first-order IIR filter
from scipy, a fixed-state softmax read), invariances and bounds.
"""
import math

import numpy as np
import pytest
import scipy.signal
import scipy.special

from oracle import bruteforce, chunkwise

RNG = np.random.default_rng(1234)


def _rand_gsa(B, H, T, dk, dv, m, g_scale=1.0, g_shift=0.0, init=False, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk)) / math.sqrt(dk)
    k = r.standard_normal((B, H, T, dk)) / math.sqrt(dk)
    v = r.standard_normal((B, H, T, dv)) / math.sqrt(dk)
    g = r.standard_normal((B, H, T, m)) * g_scale + g_shift
    k0 = v0 = None
    if init:
        k0 = r.standard_normal((B, H, m, dk)) * 0.3
        v0 = r.standard_normal((B, H, m, dv)) * 0.3
    return q, k, v, g, k0, v0


def _rel(x, y):
    den = np.max(np.abs(y))
    return np.max(np.abs(x - y)) / (den if den > 0 else 1.0)


# ---------------------------------------------------------------- P1 chunk form
@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 64])
def test_gsa_recurrent_equals_chunkwise(oracle_mod, C):
    for T in sorted({1, max(C - 1, 1), C, C + 1, 3 * C + 5}):
        q, k, v, g, k0, v0 = _rand_gsa(1, 2, T, 8, 6, 5, init=(T % 2 == 1), seed=T + C)
        ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
        o, kf, vf = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=C)
        assert _rel(ref["o"], o) < 1e-12, (C, T)
        assert _rel(ref["kf"], kf) < 1e-12, (C, T)
        assert _rel(ref["vf"], vf) < 1e-12, (C, T)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_gla_recurrent_equals_chunkwise(oracle_mod, C):
    for T in sorted({1, max(C - 1, 1), C, C + 1, 2 * C + 7}):
        r = np.random.default_rng(T * 7 + C)
        q, k = r.standard_normal((2, 1, 2, T, 8)) / 3
        v = r.standard_normal((1, 2, T, 5)) / 3
        g = r.standard_normal((1, 2, T, 8))
        s0 = r.standard_normal((1, 2, 8, 5)) if T % 2 else None
        ref = oracle_mod.gla_fwd(q, k, v, g, s0, tau=16.0)
        o, sf = chunkwise.gla_fwd(q, k, v, g, s0, tau=16.0, C=C)
        assert _rel(ref["o"], o) < 1e-12
        assert _rel(ref["sf"], sf) < 1e-12


@pytest.mark.parametrize("C,Cs", [(64, 16), (16, 4), (32, 5)])
def test_gsa_secondary_chunking_equals_recurrence(oracle_mod, C, Cs):
    """App. A.1's secondary chunking (sub-chunks of Cs tokens met through the
    first token of the query's sub-chunk, pairwise decays inside a sub-chunk)
    reproduces the recurrence, with alpha = 0 / 1 tokens and two slots at
    g ~ N(-30, 1), whose 16-token decay (~2^-86) is far below what a single
    64-token factorisation could hold."""
    q, k, v, g, k0, v0 = _rand_gsa(1, 2, 3 * C + 11, 8, 6, 5, init=True, seed=C + Cs)
    g[..., :2] -= 30.0
    g[0, 0, 3, :] = -np.inf
    g[0, 1, 10:14, 2] = np.inf
    g[0, 0, C + 1, 1] = -np.inf
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
    o, kf, vf = chunkwise.gsa_fwd_secondary(q, k, v, g, k0, v0, tau=8.0, C=C, Cs=Cs)
    assert _rel(ref["o"], o) < 1e-12
    assert _rel(ref["kf"], kf) < 1e-12
    assert _rel(ref["vf"], vf) < 1e-12


def test_gsa_chunkwise_extreme_gates(oracle_mod):
    """alpha = 0 and alpha = 1 tokens mixed in (g = -inf / +inf, and +-30)."""
    q, k, v, g, k0, v0 = _rand_gsa(1, 1, 70, 8, 8, 6, g_scale=3.0, init=True, seed=5)
    g[0, 0, 3, :] = -np.inf
    g[0, 0, 10:14, 2] = np.inf
    g[0, 0, 20, 1] = -30.0
    g[0, 0, 40:45, 4] = 30.0
    g[0, 0, 66, 0] = -np.inf
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
    assert np.all(np.isfinite(ref["o"]))
    for C in (4, 16, 64):
        o, kf, vf = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=C)
        assert _rel(ref["o"], o) < 1e-12
        assert _rel(ref["kf"], kf) < 1e-12
        assert _rel(ref["vf"], vf) < 1e-12


# ------------------------------------------------------------ P6 brute force
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_gsa_bruteforce(oracle_mod, T):
    q, k, v, g, k0, v0 = _rand_gsa(1, 1, T, 4, 3, 5, init=True, seed=T)
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
    o = bruteforce.gsa_unit(q[0, 0], k[0, 0], v[0, 0], g[0, 0], k0[0, 0], v0[0, 0], tau=8.0)
    assert _rel(ref["o"][0, 0], o) < 1e-12
    ref0 = oracle_mod.gsa_fwd(q, k, v, g, tau=3.0)
    o0 = bruteforce.gsa_unit(q[0, 0], k[0, 0], v[0, 0], g[0, 0], tau=3.0)
    assert _rel(ref0["o"][0, 0], o0) < 1e-12


@pytest.mark.parametrize("T", [1, 3, 8])
def test_gla_bruteforce(oracle_mod, T):
    r = np.random.default_rng(T)
    q, k = r.standard_normal((2, 1, 1, T, 4))
    v = r.standard_normal((1, 1, T, 3))
    g = r.standard_normal((1, 1, T, 4)) * 2
    s0 = r.standard_normal((1, 1, 4, 3))
    ref = oracle_mod.gla_fwd(q, k, v, g, s0, tau=16.0)
    o = bruteforce.gla_unit(q[0, 0], k[0, 0], v[0, 0], g[0, 0], s0[0, 0], tau=16.0)
    assert _rel(ref["o"][0, 0], o) < 1e-12


# ------------------------------------------------------------- P2 alpha = 1
def test_gla_alpha_one_is_linear_attention(oracle_mod):
    """g = +inf gives alpha = 1: plain linear attention without normaliser,
    o = tril(Q K^T) V + Q S0 (Sec. 2.2, App. A)."""
    r = np.random.default_rng(3)
    T, dk, dv = 37, 6, 5
    q, k = r.standard_normal((2, 1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    s0 = r.standard_normal((1, 1, dk, dv))
    g = np.full((1, 1, T, dk), np.inf)
    ref = oracle_mod.gla_fwd(q, k, v, g, s0, tau=16.0)
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    expect = np.tril(Q @ K.T) @ V + Q @ s0[0, 0]
    assert _rel(ref["o"][0, 0], expect) < 1e-12
    assert _rel(ref["sf"][0, 0], s0[0, 0] + K.T @ V) < 1e-12


def test_gsa_alpha_one_freezes_state(oracle_mod):
    """alpha = 1 means no write (1 - alpha = 0): o_t = V0^T softmax(K0 q_t);
    from a zero state the output is exactly 0."""
    q, k, v, g, k0, v0 = _rand_gsa(2, 1, 19, 7, 4, 6, init=True, seed=9)
    g[:] = np.inf
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
    for b in range(2):
        s = scipy.special.softmax(q[b, 0] @ k0[b, 0].T, axis=-1)
        assert _rel(ref["o"][b, 0], s @ v0[b, 0]) < 1e-13
    zero = oracle_mod.gsa_fwd(q, k, v, g, tau=8.0)
    assert np.all(zero["o"] == 0.0)


def test_gla_constant_decay_is_retention(oracle_mod):
    """A time- and dimension-independent decay gamma reduces GLA to the
    RetNet form o = (D * tril(Q K^T)) V with D[t, j] = gamma^(t-j) (Sec. 2.3)."""
    r = np.random.default_rng(11)
    T, dk, dv, tau = 29, 5, 4, 16.0
    q, k = r.standard_normal((2, 1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    g = np.full((1, 1, T, dk), 0.7)
    gamma = scipy.special.expit(0.7) ** (1.0 / tau)
    t = np.arange(T)
    D = np.tril(np.power(gamma, (t[:, None] - t[None, :]).clip(min=0)))
    ref = oracle_mod.gla_fwd(q, k, v, g, tau=tau)
    expect = (D * (q[0, 0] @ k[0, 0].T)) @ v[0, 0]
    assert _rel(ref["o"][0, 0], expect) < 1e-12


# --------------------------------------------------------- P3 softmax link
def test_slot_softmax_rows_sum_to_one(oracle_mod):
    q, k, v, g, k0, v0 = _rand_gsa(2, 3, 50, 16, 16, 12, init=True, seed=2)
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, want_scores=True)
    assert np.max(np.abs(ref["s"].sum(-1) - 1.0)) < 1e-14
    assert np.all(ref["s"] > 0)
    # s is the softmax of the raw slot scores, and o = Vt^T s with the score
    # from the state read after the update (checked by the brute-force pin).
    assert _rel(ref["s"], scipy.special.softmax(ref["z"], axis=-1)) < 1e-14


# ---------------------------------------------------------- P4 alpha -> 0
def test_gsa_alpha_zero_copies_value(oracle_mod):
    """alpha = 0: every slot is overwritten with the current k and v, the slot
    softmax is uniform and o_t = v_t exactly."""
    q, k, v, g, k0, v0 = _rand_gsa(1, 2, 23, 8, 8, 5, init=True, seed=4)
    g[:] = -np.inf
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, want_scores=True)
    assert _rel(ref["o"], v) < 1e-15
    assert np.allclose(ref["s"], 1.0 / 5, rtol=0, atol=1e-15)
    g[:] = -400.0   # alpha = sigmoid(-400)^(1/8) = e^-50
    near = oracle_mod.gsa_fwd(q, k, v, g, k0, v0)
    assert _rel(near["o"], v) < 1e-15


# -------------------------------------------------------------- P5 m = 1
def test_gsa_single_slot_is_gated_ema(oracle_mod):
    """m = 1: the softmax over one slot is 1, so o_t is the slot's value row,
    a first-order IIR filter of v with pole alpha (here constant in time),
    independent of q and k."""
    r = np.random.default_rng(8)
    T, d = 64, 6
    q, k = r.standard_normal((2, 1, 1, T, d))
    v = r.standard_normal((1, 1, T, d))
    g = np.full((1, 1, T, 1), -0.4)
    alpha = scipy.special.expit(-0.4) ** (1 / 8.0)
    ref = oracle_mod.gsa_fwd(q, k, v, g, tau=8.0)
    expect = scipy.signal.lfilter([1.0 - alpha], [1.0, -alpha], v[0, 0], axis=0)
    assert _rel(ref["o"][0, 0], expect) < 1e-12
    other = oracle_mod.gsa_fwd(q * 5.0, k[..., ::-1].copy(), v, g, tau=8.0)
    assert np.array_equal(other["o"], ref["o"])


# ------------------------------------------------ P7 slot permutation
def test_gsa_slot_permutation_invariance(oracle_mod):
    q, k, v, g, k0, v0 = _rand_gsa(1, 1, 33, 8, 8, 7, init=True, seed=6)
    perm = np.random.default_rng(0).permutation(7)
    a = oracle_mod.gsa_fwd(q, k, v, g, k0, v0)
    b = oracle_mod.gsa_fwd(q, k, v, g[..., perm].copy(), k0[:, :, perm].copy(),
                           v0[:, :, perm].copy())
    assert _rel(b["o"], a["o"]) < 1e-13
    assert _rel(b["kf"], a["kf"][:, :, perm]) < 1e-13


# ---------------------------------------------------------- P8 bound
def test_gsa_output_bounded_by_values(oracle_mod):
    q, k, v, g, _, _ = _rand_gsa(2, 2, 80, 8, 8, 6, g_scale=3.0, seed=10)
    o = oracle_mod.gsa_fwd(q * 20, k, v, g)["o"]
    vmax = np.maximum.accumulate(np.abs(v).max(-1), axis=2)
    assert np.all(np.abs(o).max(-1) <= vmax * (1 + 1e-12))


# --------------------------------------------- P9 state hand-off, decode
def test_gsa_split_handoff_and_decode_chain(oracle_mod):
    q, k, v, g, k0, v0 = _rand_gsa(2, 2, 41, 8, 6, 5, init=True, seed=12)
    full = oracle_mod.gsa_fwd(q, k, v, g, k0, v0)
    T1 = 17
    a = oracle_mod.gsa_fwd(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1], k0, v0)
    b = oracle_mod.gsa_fwd(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:],
                           a["kf"], a["vf"])
    assert _rel(np.concatenate([a["o"], b["o"]], axis=2), full["o"]) < 1e-14
    assert _rel(b["kf"], full["kf"]) < 1e-14
    ks, vs = k0.copy(), v0.copy()
    for t in range(41):
        o, ks, vs = oracle_mod.gsa_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t],
                                               ks, vs)
        assert _rel(o, full["o"][:, :, t]) < 1e-14
    assert _rel(ks, full["kf"]) < 1e-14 and _rel(vs, full["vf"]) < 1e-14


# --------------------------------------------------- P10 unit permutation
def test_units_are_independent(oracle_mod):
    q, k, v, g, k0, v0 = _rand_gsa(3, 2, 20, 8, 8, 4, init=True, seed=13)
    a = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, nthreads=4)
    idx = [2, 0, 1]
    b = oracle_mod.gsa_fwd(q[idx], k[idx], v[idx], g[idx], k0[idx], v0[idx], nthreads=1)
    assert np.array_equal(b["o"], a["o"][idx])


def test_gla_split_handoff(oracle_mod):
    r = np.random.default_rng(14)
    q, k, g = r.standard_normal((3, 1, 2, 30, 6))
    v = r.standard_normal((1, 2, 30, 4))
    full = oracle_mod.gla_fwd(q, k, v, g)
    a = oracle_mod.gla_fwd(q[:, :, :11], k[:, :, :11], v[:, :, :11], g[:, :, :11])
    b = oracle_mod.gla_fwd(q[:, :, 11:], k[:, :, 11:], v[:, :, 11:], g[:, :, 11:], a["sf"])
    assert _rel(np.concatenate([a["o"], b["o"]], 2), full["o"]) < 1e-14


# --------------------------------------------------- P10 128 slots
def test_gsa_128_slots(oracle_mod):
    """At m = 128 (the largest slot count of the pages' throughput table):
    the recurrence equals the numpy chunk form, whose softmax spans all 128
    slots at once, and permuting the slots (across the two 64-slot halves the
    GPU path splits them into) permutes the states and leaves o unchanged."""
    q, k, v, g, k0, v0 = _rand_gsa(1, 2, 150, 16, 12, 128, init=True, seed=12)
    ref = oracle_mod.gsa_fwd(q, k, v, g, k0, v0, tau=8.0)
    o, kf, vf = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=64)
    assert _rel(ref["o"], o) < 1e-12 and _rel(ref["kf"], kf) < 1e-12 and _rel(ref["vf"], vf) < 1e-12
    perm = np.concatenate([np.arange(64, 128), np.arange(64)])[np.random.default_rng(1).permutation(128)]
    b = oracle_mod.gsa_fwd(q, k, v, g[..., perm].copy(), k0[:, :, perm].copy(), v0[:, :, perm].copy())
    assert _rel(b["o"], ref["o"]) < 1e-13
    assert _rel(b["vf"], ref["vf"][:, :, perm]) < 1e-13
