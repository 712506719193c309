"""GPU parity of the recurrent GLA step (gla_decode_step) against the float64
oracle's GLA recurrence run for one token from the given state, and the
prefill -> decode chain for GLA: gla_fwd's final state continued token by
token equals one forward over the whole sequence.  Bar: 2e-2 (bf16) / 1e-4
(float32) on o, 1e-5 on the state."""
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


@pytest.mark.parametrize("gate", ["logit", "log_decay"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_gla_decode_step(gsa, torch, gate, dtype, d):
    N, H = 5, 3
    inp = synth.gla_inputs(N, H, 1, d, d, dtype=dtype, seed=d + 1, init_std=0.3,
                           log_decay_scale=0.06 if gate == "log_decay" else None)
    x = inp["g"].f64.copy()
    x[0, 0, 0, :4] = np.inf if gate == "logit" else 0.0       # alpha = 1
    x[1, 0, 0, :4] = -np.inf                                    # alpha = 0
    inp["g"] = synth.stored(x, dtype)
    tok = {n: to_dev(inp[n], torch)[:, :, 0].contiguous() for n in "qkvg"}
    s = to_dev(inp["s0"], torch).clone()
    o = gsa.gla_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], s, tau=16.0, gate=gate)
    torch.cuda.synchronize()
    ref = oracle.gla_fwd(*(inp[n].f64 for n in "qkvg"), inp["s0"].f64, tau=16.0, gate=gate)
    eo, es = rel_err(to_np(o), ref["o"][:, :, 0]), rel_err(to_np(s), ref["sf"])
    print("gla decode %s %s d%d: o %.2e s %.2e" % (gate, dtype, d, eo, es))
    assert eo <= TOL[dtype] and es <= 1e-5


def test_gla_prefill_then_decode(gsa, torch):
    """gla_fwd over the first 100 tokens, then 20 decode steps from its final
    state, against one oracle forward over all 120 tokens."""
    inp = synth.gla_inputs(2, 2, 120, 128, 128, dtype="bf16", seed=50, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    s0 = to_dev(inp["s0"], torch)
    T1 = 100
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, s = gsa.gla_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1), s0, tau=16.0,
                        final_state=True)
    outs = [gsa.gla_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                g[:, :, t].contiguous(), s, tau=16.0) for t in range(T1, 120)]
    torch.cuda.synchronize()
    ref = oracle.gla_fwd(*(inp[n].f64 for n in "qkvg"), inp["s0"].f64, tau=16.0)
    o = np.concatenate([to_np(o1), np.stack([to_np(x) for x in outs], axis=2)], axis=2)
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(to_np(s), ref["sf"]) <= TOL["bf16"]


def test_gla_decode_workload(gsa, torch):
    """The decode batch's shape (256 sequences x 16 heads, d = 128; one state of
    64 KB per unit), a sample of units against the oracle."""
    N, H, d = 256, 16, 128
    inp = synth.gla_inputs(N, H, 1, d, d, dtype="bf16", seed=51, init_std=0.1)
    tok = {n: to_dev(inp[n], torch)[:, :, 0].contiguous() for n in "qkvg"}
    s = to_dev(inp["s0"], torch)
    o = gsa.gla_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], s, tau=16.0)
    torch.cuda.synchronize()
    idx = np.array([0, 1000, N * H - 1])
    f = lambda a: a.reshape(-1, *a.shape[2:])[idx][:, None]
    ref = oracle.gla_fwd(*(f(inp[n].f64) for n in "qkvg"), f(inp["s0"].f64), tau=16.0)
    eo = rel_err(to_np(o).reshape(-1, d)[idx][:, None, None], ref["o"])
    es = rel_err(to_np(s).reshape(-1, d, d)[idx][:, None], ref["sf"])
    assert eo <= TOL["bf16"] and es <= 1e-5
