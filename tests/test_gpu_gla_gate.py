"""GPU parity of the GLA forward with the gate given directly as per-token
log-decays (gla_fwd_ex with GSA_GATE_LOG_DECAY) against the float64 oracle on
the same seeded stored inputs.  Bar: max |x - y| / max |y| per output tensor,
1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with float32 state."""
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


def _check(gsa, torch, inp, dtype, cps=0, units=None, label=""):
    q, k, v, g = (to_dev(inp[x], torch) for x in "qkvg")
    s0 = to_dev(inp["s0"], torch)
    o, sf = gsa.gla_fwd(q, k, v, g, s0, tau=16.0, final_state=True, chunks_per_segment=cps,
                        gate="log_decay")
    torch.cuda.synchronize()
    f = (lambda a: a) if units is None else (lambda a: a.reshape(-1, *a.shape[2:])[units][:, None])
    ref = oracle.gla_fwd(*(f(inp[x].f64) for x in "qkvg"), None if inp["s0"] is None else f(inp["s0"].f64),
                         nthreads=oracle.max_threads(), gate="log_decay")
    eo, es = rel_err(f(to_np(o)), ref["o"]), rel_err(f(to_np(sf)), ref["sf"])
    print("gla log-decay %s %s cps=%d: o %.2e sf %.2e" % (label, dtype, cps, eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_gla_log_decay_shapes(gsa, torch, T, dtype, d):
    inp = synth.gla_inputs(2, 2, T, d, d, dtype=dtype, seed=T + d, init_std=0.1, log_decay_scale=0.06)
    _check(gsa, torch, inp, dtype, label="B2 H2 T%d d%d" % (T, d))


@pytest.mark.parametrize("cps", [1, 2, 3, 100])
def test_gla_log_decay_segmentations(gsa, torch, cps):
    inp = synth.gla_inputs(1, 3, 64 * 7 + 5, 128, 128, dtype="bf16", seed=3, init_std=0.1,
                           log_decay_scale=0.06)
    _check(gsa, torch, inp, "bf16", cps=cps, label="B1 H3 T453")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_gla_log_decay_exact_path(gsa, torch, dtype, d):
    """Strong decays (a whole chunk far below the factorised
    form's floor), alpha = 0 (-inf) and
    positive entries (taken as 0) send chunks through the exact recurrence."""
    inp = synth.gla_inputs(1, 2, 260, d, d, dtype=dtype, seed=9, init_std=0.1, log_decay_scale=0.06)
    x = inp["g"].f64.copy()
    x[..., 64:128, :] = -3.0
    x[..., 10, :] = -np.inf
    x[..., 150:160, 5] = 0.5
    x[..., 200, :7] = -np.inf
    inp["g"] = synth.stored(x, inp["g"].dtype)
    for cps in (0, 1):
        _check(gsa, torch, inp, dtype, cps=cps, label="strong decays")


def test_gla_log_decay_full_workload_sampled_units(gsa, torch):
    w = synth.WORKLOADS["gla_bf16_T4096_log_decay"]
    inp = synth.gla_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], dtype=w["dtype"], seed=0,
                           qkv_scale=w["qkv_scale"], log_decay_scale=w["log_decay_scale"])
    _check(gsa, torch, inp, "bf16", units=np.array([0, 41, 99, w["B"] * w["H"] - 1]),
           label="B8 H16 T4096 (sampled units)")


def test_gate_code_logit_matches_plain_entry_point(gsa, torch):
    inp = synth.gla_inputs(2, 2, 300, 128, 128, dtype="bf16", seed=5)
    q, k, v, g = (to_dev(inp[x], torch) for x in "qkvg")
    o1, _ = gsa.gla_fwd(q, k, v, g)
    o2, _ = gsa.gla_fwd(q, k, v, g, gate="logit")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
