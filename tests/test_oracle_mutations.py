"""The pins must have teeth: plant plausible mistakes in a private copy of the
C oracle (compiled to a temporary library on the CPU) and check that every
mutant fails at least one pin that the real oracle passes.  The committed
oracle source is never modified."""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.special

from oracle import bruteforce, chunkwise
from tests import test_oracle_bwd

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "gsa_oracle.c")

# (name, original text, planted mistake)
MUTATIONS = [
    ("write_not_coupled", "double w = -expm1(la);", "double w = 1.0;"),
    ("write_is_alpha", "double w = -expm1(la);", "double w = a;"),
    ("exclusive_read", "Kc[x] = a * Kc[x] + w * kt[x];\n            acc += Kc[x] * qt[x];",
     "acc += Kc[x] * qt[x];\n            Kc[x] = a * Kc[x] + w * kt[x];"),
    ("logsig_sign", "return (x < 0.0 ? x : 0.0) - log1p(exp(-fabs(x)));",
     "return (x < 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));"),
    ("tau_multiplies", "double la = log_sigmoid(gt[c]) / tau;",
     "double la = log_sigmoid(gt[c]) * tau;"),
    ("softmax_unnormalised", "s[c] /= sum;", "s[c] /= 1.0;"),
    ("output_transposed", "acc += V[c * dv + x] * s[c];", "acc += V[x * dv + c] * s[c];"),
    ("value_decay_skipped", "Vc[x] = a * Vc[x] + w * vt[x];", "Vc[x] = Vc[x] + w * vt[x];"),
    ("gla_scalar_gate", "double a = gate_mode == 0 ? exp(log_sigmoid(gt[x]) / tau)",
     "double a = gate_mode == 0 ? exp(log_sigmoid(gt[0]) / tau)"),
    # GLA gate given as log-decays
    ("gla_logdecay_sign", "exp(gt[x] < 0.0 ? gt[x] : 0.0)", "exp(gt[x] < 0.0 ? -gt[x] : 0.0)"),
    ("gla_logdecay_unclamped", "exp(gt[x] < 0.0 ? gt[x] : 0.0)", "exp(gt[x])"),
    ("gla_logdecay_as_logit", ": exp(gt[x] < 0.0 ? gt[x] : 0.0);", ": exp(log_sigmoid(gt[x]) / tau);"),
    ("gla_read_before_write", "Sx[y] = a * Sx[y] + kt[x] * vt[y];",
     "Sx[y] = a * Sx[y] + kt[x] * vt[y] * (t > 0);"),
    # slot read non-linearities of the ablation study (Table 2)
    ("swish_sigmoid_sign", "return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    ("relu_leaky", "return x > 0.0 ? x : 0.0;", "return x > 0.0 ? x : 0.01 * x;"),
    ("relu2_not_squared", "return x > 0.0 ? x * x : 0.0;", "return x > 0.0 ? x : 0.0;"),
    ("read_codes_shifted", "s[c] = slot_fn(z[c], act);", "s[c] = slot_fn(z[c], act + 1);"),
    ("read_of_scaled_scores", "s[c] = slot_fn(z[c], act);", "s[c] = slot_fn(z[c] * 0.5, act);"),
    ("bwd_softmax_jacobian_unshifted", "st[c] * (ds[c] - sds)", "st[c] * ds[c]"),
    ("bwd_swish_grad_without_product_rule", "return sg * (1.0 + x * (1.0 - sg));", "return sg;"),
    ("bwd_relu2_grad_halved", "return x > 0.0 ? 2.0 * x : 0.0;", "return x > 0.0 ? x : 0.0;"),
    ("bwd_elementwise_read_grad_as_softmax", ": slot_grad(Z[t * m + c], act) * ds[c];", ": st[c] * ds[c];"),
    ("bwd_read_of_previous_state", "acc += Vn[c * d_v + x] * dOt[x];", "acc += Vp[c * d_v + x] * dOt[x];"),
    ("bwd_gate_of_new_state", "da += dK[c * d_k + x] * (Kp[c * d_k + x] - kt[x]);",
     "da += dK[c * d_k + x] * (Kn[c * d_k + x] - kt[x]);"),
    ("bwd_adjoint_decayed_by_write", "dK[c * d_k + x] *= a;", "dK[c * d_k + x] *= w;"),
    ("bwd_gate_chain_without_alpha", "dg[row * m + c] = da * a * sig_neg / tau;",
     "dg[row * m + c] = da * sig_neg / tau;"),
    ("bwd_value_adjoint_after_read", "dV[c * d_v + x] += st[c] * dOt[x];", "dV[c * d_v + x] += 0.0;"),
]


def _build(tmp_path, text, name):
    c = tmp_path / (name + ".c")
    c.write_text(text)
    so = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(c), "-lm"])
    lib = ctypes.CDLL(str(so))
    P, L, D, I = ctypes.c_void_p, ctypes.c_long, ctypes.c_double, ctypes.c_int
    lib.oracle_gsa_fwd.argtypes = [P] * 11 + [L] * 6 + [D, I]
    lib.oracle_gla_fwd.argtypes = [P] * 7 + [L] * 5 + [D, I]
    lib.oracle_gsa_fwd_nl.argtypes = [P] * 11 + [L] * 6 + [D, I, I]
    lib.oracle_gla_fwd_gm.argtypes = [P] * 7 + [L] * 5 + [D, I, I]
    lib.oracle_gsa_bwd.argtypes = [P] * 15 + [L] * 6 + [D, I]
    lib.oracle_gsa_bwd_nl.argtypes = [P] * 15 + [L] * 6 + [D, I, I]
    return lib


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _gsa(lib, q, k, v, g, k0=None, v0=None, tau=8.0, act=None):
    B, H, T, dk = q.shape
    dv, m = v.shape[-1], g.shape[-1]
    o = np.empty((B, H, T, dv))
    kf = np.empty((B, H, m, dk))
    vf = np.empty((B, H, m, dv))
    if act is None:
        rc = lib.oracle_gsa_fwd(_p(q), _p(k), _p(v), _p(g), _p(k0), _p(v0), _p(o), _p(kf),
                                _p(vf), None, None, B, H, T, dk, dv, m, tau, 1)
    else:
        rc = lib.oracle_gsa_fwd_nl(_p(q), _p(k), _p(v), _p(g), _p(k0), _p(v0), _p(o), _p(kf),
                                   _p(vf), None, None, B, H, T, dk, dv, m, tau, act, 1)
    assert rc == 0
    return o, kf, vf


def _gla(lib, q, k, v, g, s0=None, tau=16.0):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, H, T, dv))
    sf = np.empty((B, H, dk, dv))
    assert lib.oracle_gla_fwd(_p(q), _p(k), _p(v), _p(g), _p(s0), _p(o), _p(sf),
                              B, H, T, dk, dv, tau, 1) == 0
    return o, sf


def _rel(x, y):
    d = np.max(np.abs(y))
    return np.max(np.abs(x - y)) / (d if d > 0 else 1.0)


def _pins_pass(lib):
    """A compact run of the pins; True when all hold."""
    r = np.random.default_rng(77)
    T, d, m = 21, 6, 6          # m == dv keeps every planted index in bounds
    q, k = r.standard_normal((2, 1, 1, T, d)) / 2
    v = r.standard_normal((1, 1, T, d)) / 2
    g = r.standard_normal((1, 1, T, m)) * 1.5
    k0 = r.standard_normal((1, 1, m, d)) * 0.3
    v0 = r.standard_normal((1, 1, m, d)) * 0.3
    ok = True
    o, kf, vf = _gsa(lib, q, k, v, g, k0, v0)
    oc, kfc, vfc = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=8)
    ok &= _rel(o, oc) < 1e-12 and _rel(kf, kfc) < 1e-12 and _rel(vf, vfc) < 1e-12
    ob = bruteforce.gsa_unit(q[0, 0, :6], k[0, 0, :6], v[0, 0, :6], g[0, 0, :6],
                             k0[0, 0], v0[0, 0], tau=8.0)
    o6, _, _ = _gsa(lib, q[:, :, :6].copy(), k[:, :, :6].copy(), v[:, :, :6].copy(),
                    g[:, :, :6].copy(), k0, v0)
    ok &= _rel(o6[0, 0], ob) < 1e-12
    # alpha = 1 with a given state: o_t = V0^T softmax(K0 q_t)
    ginf = np.full_like(g, np.inf)
    o1, _, _ = _gsa(lib, q, k, v, ginf, k0, v0)
    ok &= _rel(o1[0, 0], scipy.special.softmax(q[0, 0] @ k0[0, 0].T, -1) @ v0[0, 0]) < 1e-13
    # GLA pins: chunkwise, brute force, alpha = 1 linear attention
    gg = r.standard_normal((1, 1, T, d))
    s0 = r.standard_normal((1, 1, d, d))
    og, sfg = _gla(lib, q, k, v, gg, s0)
    ogc, sfgc = chunkwise.gla_fwd(q, k, v, gg, s0, tau=16.0, C=8)
    ok &= _rel(og, ogc) < 1e-12 and _rel(sfg, sfgc) < 1e-12
    ola, _ = _gla(lib, q, k, v, np.full_like(gg, np.inf))
    ok &= _rel(ola[0, 0], np.tril(q[0, 0] @ k[0, 0].T) @ v[0, 0]) < 1e-12
    # GLA with log-decays given directly (a few positive entries, taken as 0),
    # against the numpy chunk form, which takes log-decays as they are
    la = -np.abs(r.standard_normal((1, 1, T, d))) * 0.3
    la[0, 0, 3, 1] = 0.2
    la[0, 0, 9, :2] = -np.inf
    ol = np.empty((1, 1, T, d))
    sl = np.empty((1, 1, d, d))
    assert lib.oracle_gla_fwd_gm(_p(q), _p(k), _p(v), _p(la), _p(s0), _p(ol), _p(sl), 1, 1, T, d, d,
                                 16.0, 1, 1) == 0
    olc, slc = chunkwise.gla_key_decay(q[0, 0], k[0, 0], v[0, 0], np.minimum(la[0, 0], 0.0),
                                       s0[0, 0], C=8)
    ok &= _rel(ol[0, 0], olc) < 1e-12 and _rel(sl[0, 0], slc) < 1e-12
    # the element-wise slot reads against the numpy chunk form
    for act, name in ((1, "identity"), (2, "swish"), (3, "relu"), (4, "relu2")):
        on, _, _ = _gsa(lib, q, k, v, g, k0, v0, act=act)
        oc, _, _ = chunkwise.gsa_fwd(q, k, v, g, k0, v0, tau=8.0, C=8, nonlinearity=name)
        ok &= _rel(on, oc) < 1e-12
    # the backward against central differences of this library's forward
    ok &= _bwd_pin(lib)
    return bool(ok)


def _bwd_pin(lib):
    ok = True
    for act in (0, 1, 2, 3, 4):
        def fwd(x, tau):
            return _gsa(lib, x["q"], x["k"], x["v"], x["g"], x["k0"], x["v0"], tau=tau,
                        act=None if act == 0 else act)

        for seed, T in ((3, 9), (4, 1)):
            x, w = test_oracle_bwd.draw(1, 1, T, 5, 5, 4, seed=seed)
            B, H, _, dk = x["q"].shape
            dv, m = x["v"].shape[-1], x["g"].shape[-1]
            gr = {n: np.empty_like(x[n]) for n in test_oracle_bwd.NAMES}
            rc = lib.oracle_gsa_bwd_nl(*(_p(x[n]) for n in "qkvg"), _p(w["o"]), _p(x["k0"]),
                                       _p(x["v0"]), _p(w["kf"]), _p(w["vf"]),
                                       *(_p(gr[n]) for n in test_oracle_bwd.NAMES), B, H, T, dk,
                                       dv, m, 8.0, act, 1)
            ok &= rc == 0
            errs = test_oracle_bwd.directional_errors(fwd, gr, x, w, 8.0, seed=seed)
            ok &= max(errs.values()) < 1e-7
    return ok


def test_unmutated_copy_passes(tmp_path):
    assert _pins_pass(_build(tmp_path, open(SRC).read(), "orig"))


@pytest.mark.parametrize("name,orig,mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, orig, mut):
    text = open(SRC).read()
    assert orig in text, "mutation anchor missing: " + name
    lib = _build(tmp_path, text.replace(orig, mut, 1), name)
    assert not _pins_pass(lib), "planted mistake not caught: " + name
