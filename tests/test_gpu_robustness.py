"""GPU parity in numerically hard corners: gates at +-inf and +-30 in the
decode step, slot softmaxes that saturate (queries scaled up until one slot
takes nearly all the weight) in the forward and the decode step, and large
states.  Bar as elsewhere: max |x - y| / max |y| per output tensor, 2e-2 for
bf16 inputs with fp32 state, 1e-4 for float32."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32)])
def test_decode_extreme_gates(gsa, torch, dtype, d, m):
    inp = synth.decode_inputs(4, 3, d, d, m, dtype=dtype, seed=40)
    x = inp["g"].f64.copy()
    x[0, :, :8] = np.inf          # frozen slots: no write
    x[1, :, :8] = -np.inf         # overwritten slots: the state row becomes k, v
    x[2, :, 8:16] = 30.0
    x[3, :, 8:16] = -30.0
    inp["g"] = synth.stored(x, dtype)
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs)
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(*(inp[n].f64 for n in "qkvg"), inp["kstate"].f64,
                                        inp["vstate"].f64)
    assert np.all(np.isfinite(to_np(o)))
    assert rel_err(to_np(o), ro) <= TOL[dtype]
    assert rel_err(to_np(ks), rk) <= 1e-5 and rel_err(to_np(vs), rv) <= 1e-5
    # alpha = 1 leaves the slot exactly as it was; alpha = 0 writes k exactly
    assert np.array_equal(to_np(ks)[0, :, :8], inp["kstate"].f64[0, :, :8])
    assert np.allclose(to_np(ks)[1, :, :8], np.broadcast_to(inp["k"].f64[1, :, None, :], (3, 8, d)),
                       rtol=0, atol=0)


@pytest.mark.parametrize("scale", [30.0, 300.0])
def test_decode_saturated_softmax(gsa, torch, scale):
    """Queries scaled up so that the slot scores spread over tens to hundreds:
    the softmax is nearly one-hot and must not overflow."""
    inp = synth.decode_inputs(8, 4, 128, 128, 64, dtype="bf16", seed=41, state_std=1.0)
    inp["q"] = synth.stored(inp["q"].f64 * scale, "bf16")
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs)
    torch.cuda.synchronize()
    ro, _, _ = oracle.gsa_decode_step(*(inp[n].f64 for n in "qkvg"), inp["kstate"].f64,
                                      inp["vstate"].f64)
    assert np.all(np.isfinite(to_np(o)))
    assert rel_err(to_np(o), ro) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d,m,scale", [("bf16", 128, 64, 30.0), ("bf16", 128, 64, 200.0),
                                             ("f32", 64, 32, 200.0)])
def test_forward_saturated_softmax(gsa, torch, dtype, d, m, scale):
    """The chunked forward with near-one-hot slot reads (scores in the tens to
    hundreds) and a large initial state."""
    inp = synth.gsa_inputs(1, 2, 200, d, d, m, dtype=dtype, seed=42, init_std=1.0)
    inp["q"] = synth.stored(inp["q"].f64 * scale, dtype)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    for cps in (0, 1):
        o, kf, vf = gsa.gsa_fwd(q, k, v, g, k0, v0, final_state=True, chunks_per_segment=cps)
        torch.cuda.synchronize()
        ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), inp["k0"].f64, inp["v0"].f64, tau=8.0)
        on = to_np(o)
        assert np.all(np.isfinite(on))
        errs = [rel_err(on, ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"])]
        print("saturated softmax %s scale %g cps %d: %s" % (dtype, scale, cps, ["%.2e" % e for e in errs]))
        assert max(errs) <= TOL[dtype]
