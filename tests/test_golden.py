"""The fp64 oracle against hand-derived worked examples (tests/golden/).

The examples are exact rationals derived from the recurrences of "Gated Slot
Attention for Efficient Linear-Time Sequence Modeling" (Sec. 2.3 for GLA,
Sec. 3.2 for GSA); the derivation is in tests/golden/README.md.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
EX = json.load(open(os.path.join(HERE, "golden", "worked_examples.json")))


def _arr(x):
    return np.vectorize(lambda s: float(Fraction(s)), otypes=[np.float64])(np.array(x, dtype=object))


def _logit_of_pow2(e):
    p = 2.0 ** e
    return math.log(p) - math.log1p(-p)


def _gates(ex, T):
    g = np.array([_logit_of_pow2(e) for e in ex["sigmoid_of_gate_log2"]])
    return np.broadcast_to(g, (T, g.size)).copy()


def _close(x, y, tol=1e-13):
    assert np.max(np.abs(np.asarray(x) - np.asarray(y))) <= tol * max(1.0, np.max(np.abs(y)))


def test_gate_logits_give_the_stated_alphas():
    for name in ("gsa", "gla"):
        ex = EX[name]
        for e, a in zip(ex["sigmoid_of_gate_log2"], ex["alpha"]):
            sig = 1.0 / (1.0 + math.exp(-_logit_of_pow2(e)))
            assert abs(sig ** (1.0 / ex["tau"]) - float(Fraction(a))) < 1e-14


def _gsa_inputs():
    ex = EX["gsa"]
    q, k, v = (_arr(ex[n])[None, None] for n in ("q", "k", "v"))
    g = _gates(ex, q.shape[2])[None, None]
    return ex, q, k, v, g


def _softmax2(z):
    s1 = 1.0 / (1.0 + math.exp(z[0] - z[1]))
    return np.array([1.0 - s1, s1])


def test_gsa_worked_example():
    ex, q, k, v, g = _gsa_inputs()
    r = oracle.gsa_fwd(q, k, v, g, tau=ex["tau"], want_scores=True)
    z = _arr(ex["z"])
    _close(r["z"][0, 0], z)
    Vs = _arr(ex["V_after"])
    for t in range(3):
        s = _softmax2(z[t])
        _close(r["s"][0, 0, t], s)
        _close(r["o"][0, 0, t], s[0] * Vs[t][0] + s[1] * Vs[t][1])
    _close(r["kf"][0, 0], _arr(ex["K_after"])[2])
    _close(r["vf"][0, 0], Vs[2])


@pytest.mark.parametrize("T", [1, 2])
def test_gsa_worked_example_prefix_states(T):
    ex, q, k, v, g = _gsa_inputs()
    r = oracle.gsa_fwd(q[:, :, :T], k[:, :, :T], v[:, :, :T], g[:, :, :T], tau=ex["tau"])
    _close(r["kf"][0, 0], _arr(ex["K_after"])[T - 1])
    _close(r["vf"][0, 0], _arr(ex["V_after"])[T - 1])


def test_gsa_worked_example_decode_step():
    ex, q, k, v, g = _gsa_inputs()
    K2 = _arr(ex["K_after"])[1][None, None]
    V2 = _arr(ex["V_after"])[1][None, None]
    o, ks, vs = oracle.gsa_decode_step(q[:, :, 2], k[:, :, 2], v[:, :, 2], g[:, :, 2], K2, V2,
                                       tau=ex["tau"])
    z = _arr(ex["z"])[2]
    s = _softmax2(z)
    V3 = _arr(ex["V_after"])[2]
    _close(o[0, 0], s[0] * V3[0] + s[1] * V3[1])
    _close(ks[0, 0], _arr(ex["K_after"])[2])
    _close(vs[0, 0], V3)


def test_gla_worked_example():
    ex = EX["gla"]
    q, k, v = (_arr(ex[n])[None, None] for n in ("q", "k", "v"))
    g = _gates(ex, 3)[None, None]
    r = oracle.gla_fwd(q, k, v, g, tau=ex["tau"])
    _close(r["o"][0, 0], _arr(ex["o"]))
    _close(r["sf"][0, 0], _arr(ex["S_after"])[2])
    for T in (1, 2):
        rt = oracle.gla_fwd(q[:, :, :T], k[:, :, :T], v[:, :, :T], g[:, :, :T], tau=ex["tau"])
        _close(rt["sf"][0, 0], _arr(ex["S_after"])[T - 1])


@pytest.mark.parametrize("nl", ["identity", "relu", "relu2", "swish"])
def test_gsa_worked_example_read_ablations(nl):
    """The oracle's element-wise reads against the hand-derived outputs (the
    exact rationals for none / ReLU / ReLU^2, Swish formed from the stated
    scores and states)."""
    ex, q, k, v, g = _gsa_inputs()
    ref = oracle.gsa_fwd(q, k, v, g, tau=ex["tau"], want_scores=True, nonlinearity=nl)
    if nl == "swish":
        z, V = _arr(ex["z"]), _arr(ex["V_after"])
        expect = np.stack([(z[t] / (1.0 + np.exp(-z[t]))) @ V[t] for t in range(3)])
    else:
        expect = _arr(ex["o_" + nl])
    _close(ref["o"][0, 0], expect)
    _close(ref["z"][0, 0], _arr(ex["z"]))
