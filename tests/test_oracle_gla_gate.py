"""Pins for the oracle's GLA with the gate given directly as per-token
log-decays (CPU only).

GLA (Sec. 2.3 of "Gated Slot Attention for Efficient Linear-Time Sequence
Modeling") decays each key dimension of S by alpha_t; here alpha_t =
exp(min(g_t, 0)) is read from a gate vector computed elsewhere (for example
the rank-one gate of Lattice's simplified chunk recurrence) instead of from
logits.  Pinned against the numpy chunk form (which takes log-decays as
given), the logit form at log alpha = log sigmoid(g) / tau, linear attention
(alpha = 1), a RetNet-style constant decay, and the reset that alpha = 0
makes.
"""
import numpy as np
import pytest
import scipy.special

from oracle import chunkwise


def _rel(x, y):
    den = np.max(np.abs(y))
    return np.max(np.abs(x - y)) / (den if den > 0 else 1.0)


def _draw(T, dk=7, dv=5, seed=0):
    r = np.random.default_rng(seed)
    q, k = r.standard_normal((2, 1, 2, T, dk)) / 2
    v = r.standard_normal((1, 2, T, dv))
    la = -np.abs(r.standard_normal((1, 2, T, dk))) * 0.2
    s0 = r.standard_normal((1, 2, dk, dv))
    return q, k, v, la, s0


@pytest.mark.parametrize("C", [1, 8, 64])
def test_log_decay_equals_chunkwise(oracle_mod, C):
    for T in sorted({1, C, C + 1, 2 * C + 3}):
        q, k, v, la, s0 = _draw(T, seed=T + C)
        ref = oracle_mod.gla_fwd(q, k, v, la, s0 if T % 2 else None, gate="log_decay")
        for h in range(2):
            o, S = chunkwise.gla_key_decay(q[0, h], k[0, h], v[0, h], la[0, h],
                                           s0[0, h] if T % 2 else None, C=C)
            assert _rel(ref["o"][0, h], o) < 1e-12 and _rel(ref["sf"][0, h], S) < 1e-12


def test_log_decay_of_logits_is_the_logit_gate(oracle_mod):
    q, k, v, _, s0 = _draw(40, seed=3)
    g = np.random.default_rng(4).standard_normal((1, 2, 40, 7))
    tau = 16.0
    a = oracle_mod.gla_fwd(q, k, v, g, s0, tau=tau)
    b = oracle_mod.gla_fwd(q, k, v, scipy.special.log_expit(g) / tau, s0, tau=123.0,
                           gate="log_decay")
    assert _rel(b["o"], a["o"]) < 1e-13 and _rel(b["sf"], a["sf"]) < 1e-13


def test_zero_log_decay_is_linear_attention(oracle_mod):
    q, k, v, la, s0 = _draw(30, seed=5)
    ref = oracle_mod.gla_fwd(q, k, v, np.zeros_like(la), gate="log_decay")
    for h in range(2):
        assert _rel(ref["o"][0, h], np.tril(q[0, h] @ k[0, h].T) @ v[0, h]) < 1e-12
    # positive log-decays are taken as 0 (alpha <= 1)
    pos = oracle_mod.gla_fwd(q, k, v, np.full_like(la, 0.5), gate="log_decay")
    assert np.array_equal(pos["o"], ref["o"])


def test_constant_log_decay_is_retention(oracle_mod):
    T, lg = 25, -0.3
    q, k, v, la, _ = _draw(T, seed=6)
    t = np.arange(T)
    D = np.tril(np.exp(lg * (t[:, None] - t[None, :]).clip(min=0)))
    ref = oracle_mod.gla_fwd(q, k, v, np.full_like(la, lg), gate="log_decay")
    for h in range(2):
        assert _rel(ref["o"][0, h], (D * (q[0, h] @ k[0, h].T)) @ v[0, h]) < 1e-12


def test_minus_infinity_resets_the_state(oracle_mod):
    """alpha = 0 on every key dimension at token t0 forgets everything before
    it: the outputs from t0 on are those of the suffix from a zero state."""
    T, t0 = 33, 12
    q, k, v, la, s0 = _draw(T, seed=7)
    la[..., t0, :] = -np.inf
    full = oracle_mod.gla_fwd(q, k, v, la, s0, gate="log_decay")
    sl = lambda x: x[:, :, t0:].copy()
    suf = oracle_mod.gla_fwd(sl(q), sl(k), sl(v), sl(la), gate="log_decay")
    assert _rel(full["o"][:, :, t0:], suf["o"]) < 1e-14 and _rel(full["sf"], suf["sf"]) < 1e-14
