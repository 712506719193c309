"""The training pair (gsa_fwd_train keeps the segment start states,
gsa_bwd_train reads them) through the C ABI.  The kept states come from the
same state-map and scan kernels, on the same split, that gsa_bwd runs to
recompute them, so the pair's gradients are gsa_bwd's bits; the training
forward's outputs are held to the oracle (2e-2 for bf16 inputs)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, gates_regime_per_chunk, rel_err, to_dev, to_np

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


def _case(gsa, torch, B, H, T, d, m, init, final, seed, nl="softmax", qkv_scale=None, edit=None):
    inp = synth.gsa_inputs(B, H, T, d, d, m, dtype="bf16", seed=seed, qkv_scale=qkv_scale,
                           init_std=0.1 if init else None)
    if edit is not None:
        edit(inp)
    gi = synth.gsa_grad_inputs(B, H, T, d, d, m, dtype="bf16", seed=seed + 1000,
                               final_std=1.0 if final else None)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {n: to_dev(gi[n], torch) for n in ("do", "dkf", "dvf")}
    o, kf, vf, states = gsa.gsa_fwd_train(dev["q"], dev["k"], dev["v"], dev["g"], dev["k0"], dev["v0"],
                                          final_state=True, nonlinearity=nl)
    assert states.numel() >= gsa.gsa_train_states_bytes(B, H, T, d, d, m)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"])
    a = gsa.gsa_bwd_train(*args, states, dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True,
                          nonlinearity=nl)
    b = gsa.gsa_bwd(*args, dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True, nonlinearity=nl)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dk0", "dv0"), a, b):
        assert torch.equal(x, y), name
    return inp, o, kf, vf


@pytest.mark.parametrize("T", [1, 65, 200, 453])
@pytest.mark.parametrize("d,m", [(128, 64), (64, 32), (128, 128)])
def test_pair_gradients_and_forward(gsa, torch, T, d, m):
    inp, o, kf, vf = _case(gsa, torch, 2, 2, T, d, m, init=T % 2 == 1, final=True, seed=T + m)
    opt = lambda x: None if x is None else x.f64
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), opt(inp["k0"]), opt(inp["v0"]),
                         nthreads=oracle.max_threads())
    for x, y in ((o, ref["o"]), (kf, ref["kf"]), (vf, ref["vf"])):
        assert rel_err(to_np(x), y) <= TOL["bf16"]


@pytest.mark.parametrize("nl", ["swish", "relu2", "identity"])
def test_pair_elementwise_reads(gsa, torch, nl):
    _case(gsa, torch, 1, 3, 300, 128, 64, init=True, final=False, seed=7, nl=nl)


@pytest.mark.parametrize("m", [64, 128])
def test_pair_subchunk_form(gsa, torch, m):
    """The chunk / sub-chunk / exact regimes in turn through the kept-state
    pair (bit-equal to gsa_bwd) and the forward against the oracle."""
    inp, o, kf, vf = _case(gsa, torch, 2, 2, 64 * 5 + 11, 128, m, init=True, final=True, seed=31,
                           edit=gates_regime_per_chunk)
    opt = lambda x: None if x is None else x.f64
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), opt(inp["k0"]), opt(inp["v0"]),
                         nthreads=oracle.max_threads())
    for x, y in ((o, ref["o"]), (kf, ref["kf"]), (vf, ref["vf"])):
        assert rel_err(to_np(x), y) <= TOL["bf16"]


def test_pair_training_shape(gsa, torch):
    """B8 H4 T2048 d128 m64 (8 segments of 4 chunks per unit)."""
    _case(gsa, torch, 8, 4, 2048, 128, 64, init=False, final=False, seed=9, qkv_scale=1 / np.sqrt(128))


def test_pair_long_context(gsa, torch):
    """B1 H8 T16384 with states (32 segments of 8 chunks per unit)."""
    _case(gsa, torch, 1, 8, 16384, 128, 64, init=True, final=True, seed=10, qkv_scale=1 / np.sqrt(128))


def test_autograd_uses_the_pair(gsa, torch):
    """gsa_autograd's gradients equal gsa_bwd's bits (it runs the pair)."""
    inp = synth.gsa_inputs(2, 2, 200, 128, 128, 64, dtype="bf16", seed=11, init_std=0.1)
    dev = {n: to_dev(inp[n], torch).requires_grad_(True) for n in ("q", "k", "v", "g", "k0", "v0")}
    assert gsa.gsa_train_supported(dev["q"], dev["v"], dev["g"])
    o, kf, vf = gsa.gsa_autograd(dev["q"], dev["k"], dev["v"], dev["g"], dev["k0"], dev["v0"])
    w = torch.randn_like(o)
    (o * w).sum().backward()
    ref = gsa.gsa_bwd(*(dev[n].detach() for n in "qkvg"), w.to(o.dtype), dev["k0"].detach(),
                      dev["v0"].detach(), torch.zeros_like(kf), torch.zeros_like(vf), state_grads=True)
    torch.cuda.synchronize()
    for name, r in zip(("q", "k", "v", "g", "k0", "v0"), ref):
        assert torch.equal(dev[name].grad, r), name


def test_pair_rejects(gsa, torch):
    inp = synth.gsa_inputs(1, 1, 64, 128, 128, 64, dtype="bf16", seed=12)
    dev = {n: to_dev(inp[n], torch) for n in "qkvg"}
    with pytest.raises(gsa.GsaError):  # ReLU: the backward keeps its token walks
        gsa.gsa_fwd_train(dev["q"], dev["k"], dev["v"], dev["g"], nonlinearity="relu")
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    o, _, _, st = gsa.gsa_fwd_train(dev["q"], dev["k"], dev["v"], dev["g"])
    with pytest.raises(gsa.GsaError):  # states shorter than gsa_train_states_bytes
        gsa.gsa_bwd_train(dev["q"], dev["k"], dev["v"], dev["g"], torch.randn_like(o), small)
