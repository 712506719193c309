"""Pins for the oracle's GSA backward (CPU only), for the softmax read and the
element-wise reads of the ablation study (Table 2).

The backward is the gradient of the forward, so it is pinned against
numerical differentiation of the forward oracle (which its own pins tie to the
chunk form, unrolled sums and the worked examples): central differences of a
scalar loss L = <W, o> + <A, kf> + <Bv, vf> along random directions of every
input, and element by element on a tiny problem.  Exact special cases close
the gaps that differences cannot see: a gate at -inf (alpha = 0) cuts every
gradient path to earlier tokens and to the initial states, and a gate at +inf
(alpha = 1, write intensity 0) makes that token's k and v irrelevant.

GSA: Sec. 3.2-3.3 (the recurrence and its gate), App. B (training).
"""
import numpy as np
import pytest

import oracle

NAMES = ("q", "k", "v", "g", "k0", "v0")


def draw(B, H, T, dk, dv, m, seed, init=True, final=True):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal((B, H, T, dk)) / 2, k=r.standard_normal((B, H, T, dk)) / 2,
             v=r.standard_normal((B, H, T, dv)), g=r.standard_normal((B, H, T, m)) * 1.5,
             k0=r.standard_normal((B, H, m, dk)) * 0.3 if init else None,
             v0=r.standard_normal((B, H, m, dv)) * 0.3 if init else None)
    w = dict(o=r.standard_normal((B, H, T, dv)),
             kf=r.standard_normal((B, H, m, dk)) if final else None,
             vf=r.standard_normal((B, H, m, dv)) if final else None)
    return x, w


def loss(fwd, x, w, tau):
    """<W, o> + <A, kf> + <Bv, vf> through the forward oracle fwd(x, tau)."""
    o, kf, vf = fwd(x, tau)
    L = float(np.sum(w["o"] * o))
    if w["kf"] is not None:
        L += float(np.sum(w["kf"] * kf)) + float(np.sum(w["vf"] * vf))
    return L


def fwd_oracle(x, tau, nonlinearity="softmax"):
    r = oracle.gsa_fwd(x["q"], x["k"], x["v"], x["g"], x["k0"], x["v0"], tau=tau,
                       nonlinearity=nonlinearity)
    return r["o"], r["kf"], r["vf"]


def bwd_oracle(x, w, tau, nonlinearity="softmax"):
    r = oracle.gsa_bwd(x["q"], x["k"], x["v"], x["g"], w["o"], x["k0"], x["v0"], w["kf"], w["vf"],
                       tau=tau, nonlinearity=nonlinearity)
    return {n: r["d" + n] for n in NAMES}


def directional_errors(fwd, grads, x, w, tau, seed, eps=1e-5):
    """Relative error of <grad_X, U> against the central difference of the
    loss along a random U, for every input X that is present."""
    r = np.random.default_rng(seed)
    errs = {}
    for n in NAMES:
        if x[n] is None:
            continue
        u = r.standard_normal(x[n].shape)
        xp = dict(x)
        xm = dict(x)
        xp[n] = x[n] + eps * u
        xm[n] = x[n] - eps * u
        num = (loss(fwd, xp, w, tau) - loss(fwd, xm, w, tau)) / (2 * eps)
        ana = float(np.sum(grads[n] * u))
        errs[n] = abs(num - ana) / max(abs(num), 1e-3 * np.sqrt(np.sum(grads[n] ** 2)) + 1e-12)
    return errs


@pytest.mark.parametrize("T", [1, 6, 29])
@pytest.mark.parametrize("tau", [8.0, 1.0])
@pytest.mark.parametrize("init,final", [(True, True), (False, False), (True, False)])
def test_directional_derivatives(T, tau, init, final):
    x, w = draw(1, 2, T, 5, 4, 3, seed=T * 7 + int(tau), init=init, final=final)
    errs = directional_errors(fwd_oracle, bwd_oracle(x, w, tau), x, w, tau, seed=T)
    assert max(errs.values()) < 1e-7, errs


def test_every_element_by_central_differences():
    """Each entry of every gradient on a tiny problem (T 4, dk 3, dv 2, m 3)."""
    x, w = draw(1, 1, 4, 3, 2, 3, seed=11)
    tau, eps = 8.0, 1e-6
    grads = bwd_oracle(x, w, tau)
    for n in NAMES:
        num = np.empty_like(x[n])
        for idx in np.ndindex(x[n].shape):
            xp = dict(x)
            xm = dict(x)
            xp[n] = x[n].copy()
            xm[n] = x[n].copy()
            xp[n][idx] += eps
            xm[n][idx] -= eps
            num[idx] = (loss(fwd_oracle, xp, w, tau) - loss(fwd_oracle, xm, w, tau)) / (2 * eps)
        scale = np.max(np.abs(num))
        assert np.max(np.abs(grads[n] - num)) <= 1e-7 * max(scale, 1.0), n


def test_long_sequence_directional():
    """Gradients carried back over 300 tokens of 8 slots, with states."""
    x, w = draw(1, 1, 300, 16, 16, 8, seed=5)
    errs = directional_errors(fwd_oracle, bwd_oracle(x, w, 8.0), x, w, 8.0, seed=6, eps=1e-5)
    assert max(errs.values()) < 1e-6, errs


def test_reset_gate_cuts_the_past():
    """alpha = 0 on every slot at token t0: with no loss on outputs before t0,
    nothing before t0 (and no initial state) receives gradient."""
    T, t0 = 20, 9
    x, w = draw(1, 2, T, 5, 4, 3, seed=21)
    x["g"][..., t0, :] = -np.inf
    w["o"][..., :t0, :] = 0.0
    gr = bwd_oracle(x, w, 8.0)
    for n in ("q", "k", "v", "g"):
        assert np.all(gr[n][..., :t0, :] == 0.0), n
    assert np.all(gr["k0"] == 0.0) and np.all(gr["v0"] == 0.0)
    assert np.all(gr["g"][..., t0, :] == 0.0)       # d alpha / d g = 0 at alpha = 0
    assert np.any(gr["k"][..., t0, :] != 0.0)


def test_frozen_gate_ignores_the_token():
    """alpha = 1 (g = +inf) on every slot at token t1: k_t1 and v_t1 are not
    written, so their gradients and the gate's vanish; q_t1 still reads."""
    T, t1 = 15, 6
    x, w = draw(1, 2, T, 5, 4, 3, seed=22)
    x["g"][..., t1, :] = np.inf
    gr = bwd_oracle(x, w, 8.0)
    assert np.all(gr["k"][..., t1, :] == 0.0) and np.all(gr["v"][..., t1, :] == 0.0)
    assert np.all(gr["g"][..., t1, :] == 0.0)
    assert np.any(gr["q"][..., t1, :] != 0.0)


def test_batch_units_are_independent():
    x, w = draw(2, 3, 12, 4, 4, 2, seed=23)
    full = bwd_oracle(x, w, 8.0)
    for b in range(2):
        for h in range(3):
            xs = {n: None if x[n] is None else x[n][b:b + 1, h:h + 1].copy() for n in NAMES}
            ws = {n: w[n][b:b + 1, h:h + 1].copy() for n in w}
            part = bwd_oracle(xs, ws, 8.0)
            for n in NAMES:
                assert np.array_equal(part[n][0, 0], full[n][b, h]), n


@pytest.mark.parametrize("nl", ["identity", "swish", "relu", "relu2"])
@pytest.mark.parametrize("T", [1, 13])
def test_directional_derivatives_elementwise_reads(nl, T):
    """The backward of each element-wise read against central differences of
    the forward with that read."""
    x, w = draw(1, 2, T, 5, 4, 3, seed=40 + T)

    def fwd(xx, tau):
        return fwd_oracle(xx, tau, nl)
    errs = directional_errors(fwd, bwd_oracle(x, w, 8.0, nl), x, w, 8.0, seed=T + 1)
    assert max(errs.values()) < 1e-7, (nl, errs)


def test_identity_read_gradient_of_q_is_linear_map():
    """With no non-linearity and alpha = 1 (frozen states K0, V0) the output
    is o_t = V0^T K0 q_t, so dq_t = K0^T V0 dO_t exactly."""
    x, w = draw(1, 1, 7, 5, 4, 3, seed=50)
    x["g"][:] = np.inf
    gr = bwd_oracle(x, w, 8.0, "identity")
    K0, V0 = x["k0"][0, 0], x["v0"][0, 0]
    assert np.allclose(gr["q"][0, 0], w["o"][0, 0] @ V0.T @ K0, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("C", [1, 3, 8, 64])
@pytest.mark.parametrize("T", [1, 7, 20, 70])
def test_chunk_form_backward_equals_recurrent(C, T):
    """App. B's chunk-form backward (two GLA backward passes in reverse order,
    dI summed over both, the gate gradient as a reversed cumsum) gives the
    recurrent reverse-mode gradients."""
    from oracle import chunkwise
    x, w = draw(1, 2, T, 5, 4, 3, seed=80 + T + C)
    ref = bwd_oracle(x, w, 8.0)
    got = chunkwise.gsa_bwd(x["q"], x["k"], x["v"], x["g"], w["o"], x["k0"], x["v0"], w["kf"],
                            w["vf"], tau=8.0, C=C)
    for n in NAMES:
        den = max(np.max(np.abs(ref[n])), 1e-300)
        assert np.max(np.abs(got["d" + n] - ref[n])) / den < 1e-11, (n, C, T)


def test_chunk_form_backward_extreme_gates():
    """Gates at -inf / +inf inside and across chunks: the chunk form's decays
    are sums of log alpha, never differences of running sums."""
    from oracle import chunkwise
    x, w = draw(1, 1, 40, 5, 4, 3, seed=90, init=True, final=True)
    x["g"][..., 5, :] = -np.inf
    x["g"][..., 12:15, 1] = np.inf
    x["g"][..., 30, 0] = -np.inf
    ref = bwd_oracle(x, w, 8.0)
    got = chunkwise.gsa_bwd(x["q"], x["k"], x["v"], x["g"], w["o"], x["k0"], x["v0"], w["kf"],
                            w["vf"], tau=8.0, C=8)
    for n in NAMES:
        den = max(np.max(np.abs(ref[n])), 1e-300)
        assert np.all(np.isfinite(got["d" + n])), n
        assert np.max(np.abs(got["d" + n] - ref[n])) / den < 1e-11, n


def test_directional_derivatives_128_slots():
    """The backward at m = 128, with states and final-state gradients."""
    x, w = draw(1, 1, 40, 8, 6, 128, seed=17)
    errs = directional_errors(fwd_oracle, bwd_oracle(x, w, 8.0), x, w, 8.0, seed=18)
    assert max(errs.values()) < 1e-7, errs
