"""GPU parity at the size limits: the largest unit count the launch grid takes
(65535 (batch, head) units, 32767 with 128 slots), tensors of more than 2^31 elements (64-bit
offsets everywhere), and a decode batch of 131072 units; the same limits for
the backward.  The inputs are drawn
on the device with a seeded torch generator; sampled units are copied back and
checked against the float64 oracle run on exactly those stored values.

Bar: max |x - y| / max |y| per output tensor <= 2e-2 (bf16 inputs, fp32 state).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, rel_err, to_np

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


def _randn(torch, gen, shape, scale, shift=0.0):
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    x.mul_(scale).add_(shift)
    y = x.to(torch.bfloat16)
    del x
    return y


def _unit(t, u):
    """Unit u of a [B, H, ...] device tensor -> float64 [1, 1, ...] on the host."""
    flat = t.reshape(-1, *t.shape[2:])
    return to_np(flat[u])[None, None]


def _gsa_sampled(gsa, torch, B, H, T, d, m, units, cps=0, seed=0):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    sc = 1.0 / np.sqrt(d)
    q = _randn(torch, gen, (B, H, T, d), sc)
    k = _randn(torch, gen, (B, H, T, d), sc)
    v = _randn(torch, gen, (B, H, T, d), sc)
    g = _randn(torch, gen, (B, H, T, m), 1.0)
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, final_state=True, chunks_per_segment=cps)
    torch.cuda.synchronize()
    worst = 0.0
    for u in units:
        ref = oracle.gsa_fwd(_unit(q, u), _unit(k, u), _unit(v, u), _unit(g, u), tau=8.0,
                             nthreads=oracle.max_threads())
        worst = max(worst, rel_err(_unit(o, u), ref["o"]), rel_err(_unit(kf, u), ref["kf"]),
                    rel_err(_unit(vf, u), ref["vf"]))
    print("gsa B%d H%d T%d d%d m%d cps=%d units %s: worst rel err %.2e (%d elements per input)"
          % (B, H, T, d, m, cps, list(units), worst, q.numel()))
    del q, k, v, g, o, kf, vf
    torch.cuda.empty_cache()
    return worst


def test_gsa_max_units(gsa, torch):
    """65535 units (the grid's limit; one more is rejected on the host)."""
    B = 65535
    assert _gsa_sampled(gsa, torch, B, 1, 70, 64, 32, [0, 1, 32768, B - 1], seed=1) <= TOL["bf16"]


@pytest.mark.parametrize("cps", [0, 86, 64])
def test_gsa_over_2g_elements(gsa, torch, cps):
    """q, k, v of 2^31 + elements each (64 x 16 units x 16385 tokens x 128):
    row offsets past 2^31 elements; one segment per unit (cps 0), three
    segments whose two maps the output workgroups fold (cps 86), and five
    segments with the scan kernel (cps 64)."""
    B, H, T = 64, 16, 16385
    units = [0, 517, B * H - 1]
    assert _gsa_sampled(gsa, torch, B, H, T, 128, 64, units, cps=cps, seed=2) <= TOL["bf16"]


def test_gla_over_2g_elements(gsa, torch):
    B, H, T, d = 64, 16, 16385, 128
    gen = torch.Generator(device="cuda").manual_seed(3)
    sc = 1.0 / np.sqrt(d)
    q = _randn(torch, gen, (B, H, T, d), sc)
    k = _randn(torch, gen, (B, H, T, d), sc)
    v = _randn(torch, gen, (B, H, T, d), sc)
    g = _randn(torch, gen, (B, H, T, d), 1.0)
    o, sf = gsa.gla_fwd(q, k, v, g, tau=16.0, final_state=True)
    torch.cuda.synchronize()
    worst = 0.0
    for u in (0, 600, B * H - 1):
        ref = oracle.gla_fwd(_unit(q, u), _unit(k, u), _unit(v, u), _unit(g, u), tau=16.0)
        worst = max(worst, rel_err(_unit(o, u), ref["o"]), rel_err(_unit(sf, u), ref["sf"]))
    print("gla B%d H%d T%d d%d: worst rel err %.2e (%d elements per input)" % (B, H, T, d, worst, q.numel()))
    del q, k, v, g, o, sf
    torch.cuda.empty_cache()
    assert worst <= TOL["bf16"]


def test_decode_131072_units(gsa, torch):
    N, H, d, m = 8192, 16, 128, 64
    gen = torch.Generator(device="cuda").manual_seed(4)
    sc = 1.0 / np.sqrt(d)
    q = _randn(torch, gen, (N, H, d), sc)
    k = _randn(torch, gen, (N, H, d), sc)
    v = _randn(torch, gen, (N, H, d), sc)
    g = _randn(torch, gen, (N, H, m), 1.0)
    ks = torch.randn((N, H, m, d), generator=gen, device="cuda").mul_(0.1)
    vs = torch.randn((N, H, m, d), generator=gen, device="cuda").mul_(0.1)
    sample = [0, 70001, N * H - 1]
    k0 = [to_np(ks.reshape(-1, m, d)[u]) for u in sample]
    v0 = [to_np(vs.reshape(-1, m, d)[u]) for u in sample]
    o = gsa.gsa_decode_step(q, k, v, g, ks, vs)
    torch.cuda.synchronize()
    worst = 0.0
    for i, u in enumerate(sample):
        f = lambda t: to_np(t.reshape(-1, t.shape[-1])[u])[None, None]
        ro, rk, rv = oracle.gsa_decode_step(f(q), f(k), f(v), f(g), k0[i][None, None], v0[i][None, None])
        worst = max(worst, rel_err(f(o), ro))
        assert rel_err(to_np(ks.reshape(-1, m, d)[u])[None, None], rk) <= 1e-5
        assert rel_err(to_np(vs.reshape(-1, m, d)[u])[None, None], rv) <= 1e-5
    print("decode N%d H%d: worst o rel err %.2e" % (N, H, worst))
    del q, k, v, g, ks, vs, o
    torch.cuda.empty_cache()
    assert worst <= TOL["bf16"]


def _bwd_sampled(gsa, torch, B, H, T, d, m, units, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    sc = 1.0 / np.sqrt(d)
    q = _randn(torch, gen, (B, H, T, d), sc)
    k = _randn(torch, gen, (B, H, T, d), sc)
    v = _randn(torch, gen, (B, H, T, d), sc)
    g = _randn(torch, gen, (B, H, T, m), 1.0)
    do = _randn(torch, gen, (B, H, T, d), 1.0)
    grads = gsa.gsa_bwd(q, k, v, g, do)
    torch.cuda.synchronize()
    worst = 0.0
    for u in units:
        ref = oracle.gsa_bwd(_unit(q, u), _unit(k, u), _unit(v, u), _unit(g, u), _unit(do, u), tau=8.0)
        for name, x in zip(("dq", "dk", "dv", "dg"), grads[:4]):
            worst = max(worst, rel_err(_unit(x, u), ref[name]))
    print("gsa_bwd B%d H%d T%d d%d m%d units %s: worst rel err %.2e (%d elements per input)"
          % (B, H, T, d, m, list(units), worst, q.numel()))
    del q, k, v, g, do, grads
    torch.cuda.empty_cache()
    return worst


def test_bwd_max_units(gsa, torch):
    B = 65535
    assert _bwd_sampled(gsa, torch, B, 1, 70, 64, 32, [0, 1, 32768, B - 1], seed=5) <= TOL["bf16"]


def test_m128_max_units(gsa, torch):
    """128 slots run as two groups of 64, each group a unit of the launches:
    32767 (batch, head) pairs are 65534 group units, the most the grid takes
    (one pair more is rejected on the host); forward and backward."""
    B = 32767
    units = [0, 1, 16384, B - 1]
    assert _gsa_sampled(gsa, torch, B, 1, 70, 64, 128, units, seed=7) <= TOL["bf16"]
    assert _bwd_sampled(gsa, torch, B, 1, 70, 64, 128, units, seed=8) <= TOL["bf16"]


@pytest.mark.parametrize("m,B", [(64, 65535), (128, 32767)])
def test_pair_max_units(gsa, torch, m, B):
    """The training pair at the largest unit count: its kept states give
    gsa_bwd's gradients bit for bit, and its forward matches gsa_fwd's."""
    T, d = 70, 64
    gen = torch.Generator(device="cuda").manual_seed(9 + m)
    sc = 1.0 / np.sqrt(d)
    q = _randn(torch, gen, (B, 1, T, d), sc)
    k = _randn(torch, gen, (B, 1, T, d), sc)
    v = _randn(torch, gen, (B, 1, T, d), sc)
    g = _randn(torch, gen, (B, 1, T, m), 1.0)
    do = _randn(torch, gen, (B, 1, T, d), 1.0)
    o, _, _, states = gsa.gsa_fwd_train(q, k, v, g)
    o_ref, _, _ = gsa.gsa_fwd(q, k, v, g)
    a = gsa.gsa_bwd_train(q, k, v, g, do, states)
    b = gsa.gsa_bwd(q, k, v, g, do)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dg"), a[:4], b[:4]):
        assert torch.equal(x, y), name
    assert rel_err(to_np(o), to_np(o_ref)) <= TOL["bf16"]
    del q, k, v, g, do, o, o_ref, states, a, b
    torch.cuda.empty_cache()


def test_bwd_over_2g_elements(gsa, torch):
    """q, k, v, dO and the gradients of 2^31 + elements each (about 90 GB of
    device memory with the workspace)."""
    B, H, T = 64, 16, 16385
    assert _bwd_sampled(gsa, torch, B, H, T, 128, 64, [0, 517, B * H - 1], seed=6) <= TOL["bf16"]
