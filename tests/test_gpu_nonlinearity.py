"""GPU parity of the slot read non-linearity ablations (GSA Table 2: none,
Swish, ReLU, ReLU^2 in place of the slot softmax) through the C ABI's
gsa_fwd_ex / gsa_decode_step_ex, against the float64 oracle on the same seeded
stored inputs.

Bar (max |x - y| / max |y| per output tensor): 1e-4 for float32 inputs, 2e-2
for bfloat16 inputs with float32 state; decode states 1e-5 (they do not
depend on the read).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

ELEMENTWISE = ["identity", "swish", "relu", "relu2"]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def gsa(torch):
    import slot_memory_sequence_amd as m
    return m


def _opt(x):
    return None if x is None else x.f64


def _check(gsa, torch, inp, nl, dtype, tau=8.0, cps=0, label=""):
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, k0, v0, tau=tau, final_state=True, chunks_per_segment=cps,
                            nonlinearity=nl)
    torch.cuda.synchronize()
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), _opt(inp["k0"]), _opt(inp["v0"]), tau=tau,
                         nthreads=oracle.max_threads(), nonlinearity=nl)
    errs = [rel_err(to_np(o), ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"])]
    print("gsa %s %s %s cps=%d: o %.2e kf %.2e vf %.2e" % (label, nl, dtype, cps, *errs))
    assert max(errs) <= TOL[dtype], errs
    return o


@pytest.mark.parametrize("nl", ELEMENTWISE)
@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 64, 32)])
def test_gsa_nonlinearity_shapes(gsa, torch, nl, T, dtype, d, m):
    inp = synth.gsa_inputs(2, 2, T, d, d, m, dtype=dtype, seed=T + m, init_std=0.1)
    _check(gsa, torch, inp, nl, dtype, label="B2 H2 T%d d%d m%d" % (T, d, m))


@pytest.mark.parametrize("nl", ["identity", "relu2"])
@pytest.mark.parametrize("cps", [1, 2, 100])
def test_gsa_nonlinearity_segmentations(gsa, torch, nl, cps):
    """Every segment split (scan kernel, maps folded in the output kernel, one
    segment) gives the same read."""
    inp = synth.gsa_inputs(1, 3, 64 * 7 + 5, 128, 128, 64, dtype="bf16", seed=3, init_std=0.1)
    _check(gsa, torch, inp, nl, "bf16", cps=cps, label="B1 H3 T453")


def _extreme(inp):
    g = inp["g"]
    x = g.f64.copy()
    x[..., 3, :] = -np.inf
    x[..., 70:75, 2] = np.inf
    x[..., 100, :5] = -30.0
    x[..., 130:140, 7] = 30.0
    x[..., 200:260, 1] = -np.inf
    inp["g"] = synth.stored(x, g.dtype)


@pytest.mark.parametrize("nl", ELEMENTWISE)
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64)])
def test_gsa_nonlinearity_exact_path(gsa, torch, nl, dtype, d, m):
    """alpha = 0 / 1 tokens send chunks to the exact token recurrence, which
    applies the same read."""
    inp = synth.gsa_inputs(1, 2, 300, d, d, m, dtype=dtype, seed=7, init_std=0.1)
    _extreme(inp)
    for cps in (0, 1):
        _check(gsa, torch, inp, nl, dtype, cps=cps, label="extreme gates")


@pytest.mark.parametrize("nl", ELEMENTWISE)
def test_gsa_nonlinearity_subchunk_form(gsa, torch, nl):
    """Chunks in the sub-chunk form (8 slots at g ~ N(-10, 1): 64-token decay
    products ~2^-115, 16-token ~2^-29) apply the same read."""
    inp = synth.gsa_inputs(1, 2, 64 * 4 + 9, 128, 128, 64, dtype="bf16", seed=9, init_std=0.1)
    x = inp["g"].f64.copy()
    x[..., :8] = -10.0 + np.random.default_rng(4).standard_normal(x[..., :8].shape)
    inp["g"] = synth.stored(x, "bf16")
    for cps in (0, 1):
        _check(gsa, torch, inp, nl, "bf16", cps=cps, label="sub-chunk form")


@pytest.mark.parametrize("nl", ELEMENTWISE)
def test_gsa_nonlinearity_training_shape(gsa, torch, nl):
    """The training-shape workload (B8 H4 T2048 d128 m64, bf16) in the launch
    configuration the benchmark times, every unit against the oracle."""
    w = synth.WORKLOADS["gsa_bf16_train_T2048"]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"])
    _check(gsa, torch, inp, nl, "bf16", tau=w["tau"], label="B8 H4 T2048")


@pytest.mark.parametrize("nl", ELEMENTWISE)
@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32)])
def test_decode_nonlinearity(gsa, torch, nl, dtype, d, m):
    inp = synth.decode_inputs(3, 5, d, d, m, dtype=dtype, seed=m + 1)
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs, nonlinearity=nl)
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(*(inp[n].f64 for n in "qkvg"), inp["kstate"].f64,
                                        inp["vstate"].f64, nonlinearity=nl)
    eo = rel_err(to_np(o), ro)
    print("decode %s %s: o %.2e" % (nl, dtype, eo))
    assert eo <= TOL[dtype]
    assert rel_err(to_np(ks), rk) <= 1e-5 and rel_err(to_np(vs), rv) <= 1e-5


def test_decode_chain_equals_fwd_swish(gsa, torch):
    """Chained decode steps and the chunkwise forward agree under Swish."""
    inp = synth.gsa_inputs(2, 2, 70, 64, 64, 32, dtype="f32", seed=21, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    ks, vs = to_dev(inp["k0"], torch).clone(), to_dev(inp["v0"], torch).clone()
    o_fwd, kf, vf = gsa.gsa_fwd(q, k, v, g, to_dev(inp["k0"], torch), to_dev(inp["v0"], torch),
                                final_state=True, nonlinearity="swish")
    outs = [gsa.gsa_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                v[:, :, t].contiguous(), g[:, :, t].contiguous(), ks, vs,
                                nonlinearity="swish") for t in range(70)]
    torch.cuda.synchronize()
    assert rel_err(np.stack([to_np(x) for x in outs], axis=2), to_np(o_fwd)) <= 1e-5
    assert rel_err(to_np(ks), to_np(kf)) <= 1e-5 and rel_err(to_np(vs), to_np(vf)) <= 1e-5


def test_softmax_code_matches_plain_entry_point(gsa, torch):
    """gsa_fwd_ex with the softmax code runs exactly the kernels of gsa_fwd."""
    inp = synth.gsa_inputs(2, 2, 300, 128, 128, 64, dtype="bf16", seed=5)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o1, _, _ = gsa.gsa_fwd(q, k, v, g)
    o2, _, _ = gsa.gsa_fwd(q, k, v, g, nonlinearity="softmax")
    o3, _, _ = gsa.gsa_fwd(q, k, v, g, nonlinearity="relu")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and not torch.equal(o1, o3)


@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32)])
def test_gsa_data_independent_decay(gsa, torch, dtype, d, m):
    """Table 2's data-independent decay: one gate per (head, slot), the same at
    every token (an input pattern of the same kernels)."""
    inp = synth.gsa_inputs(2, 2, 200, d, d, m, dtype=dtype, seed=17, init_std=0.1)
    x = inp["g"].f64.copy()
    x[:] = x[:, :, :1, :]          # the first token's logits for every token
    inp["g"] = synth.stored(x, inp["g"].dtype)
    _check(gsa, torch, inp, "softmax", dtype, label="data-independent decay")
