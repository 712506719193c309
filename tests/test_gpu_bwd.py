"""GPU parity of the GSA backward (gsa_bwd, through the C ABI) against the
float64 oracle's reverse-mode differentiation of the token recurrence, on the
same seeded stored inputs.

Bar (max |x - y| / max |y| per gradient tensor): 1e-4 for float32 inputs,
2e-2 for bfloat16 inputs (fp32 states and accumulation, bf16 gradients out);
the initial-state gradients (always float32) are held to the input dtype's
bar as well.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, gates_fast_slots, gates_regime_per_chunk, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dk0", "dv0")


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


def _run(gsa, torch, inp, gi, tau, nl="softmax"):
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {n: to_dev(gi[n], torch) for n in ("do", "dkf", "dvf")}
    out = gsa.gsa_bwd(dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"], dev["k0"], dev["v0"],
                      ddev["dkf"], ddev["dvf"], tau=tau, state_grads=True, nonlinearity=nl)
    torch.cuda.synchronize()
    return dict(zip(GRADS, out))


def _ref(inp, gi, tau, units=None, nl="softmax"):
    """The oracle on all units, or on the listed flat unit indices."""
    def sel(x):
        if x is None:
            return None
        a = x.f64
        if units is None:
            return a
        return a.reshape(-1, *a.shape[2:])[units][:, None]
    return oracle.gsa_bwd(*(sel(inp[n]) for n in "qkvg"), sel(gi["do"]), sel(inp["k0"]),
                          sel(inp["v0"]), sel(gi["dkf"]), sel(gi["dvf"]), tau=tau,
                          nthreads=oracle.max_threads(), nonlinearity=nl)


def _compare(got, ref, dtype, label, units=None):
    errs = {}
    for n in GRADS:
        x = to_np(got[n])
        if units is not None:
            x = x.reshape(-1, *x.shape[2:])[units][:, None]
        errs[n] = rel_err(x, ref[n])
    print("gsa_bwd %s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    assert max(errs.values()) <= TOL[dtype], errs


def _check(gsa, torch, B, H, T, d, m, dtype, init, final, tau=8.0, seed=0, edit=None,
           nl="softmax"):
    inp = synth.gsa_inputs(B, H, T, d, d, m, dtype=dtype, seed=seed,
                           init_std=0.1 if init else None)
    if edit:
        edit(inp)
    gi = synth.gsa_grad_inputs(B, H, T, d, d, m, dtype=dtype, seed=seed + 1000,
                               final_std=1.0 if final else None)
    got = _run(gsa, torch, inp, gi, tau, nl)
    _compare(got, _ref(inp, gi, tau, nl=nl), dtype,
             "B%d H%d T%d d%d m%d %s init=%s final=%s %s" % (B, H, T, d, m, dtype, init, final, nl))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64)])
def test_bwd_lengths(gsa, torch, T, dtype, d, m):
    """One token, a partial chunk, an exact chunk, a ragged tail, several chunks."""
    _check(gsa, torch, 2, 2, T, d, m, dtype, init=True, final=True, seed=T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,m", [(128, 64), (64, 32), (128, 32), (64, 64)])
def test_bwd_shapes(gsa, torch, dtype, d, m):
    _check(gsa, torch, 1, 3, 150, d, m, dtype, init=True, final=True, seed=d + m)


@pytest.mark.parametrize("init,final", [(False, False), (True, False), (False, True)])
def test_bwd_optional_states(gsa, torch, init, final):
    """Zero initial states and / or no final-state gradients."""
    _check(gsa, torch, 2, 2, 130, 128, 64, "bf16", init=init, final=final, seed=7)


@pytest.mark.parametrize("which", ["k0", "v0"])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 128, 128)])
def test_bwd_one_initial_state(gsa, torch, which, dtype, d, m):
    """Only one of the two initial slot states given: the other is zero and its
    gradient is still written."""
    def drop(inp):
        inp["v0" if which == "k0" else "k0"] = None
    _check(gsa, torch, 2, 2, 64 * 3 + 11, d, m, dtype, True, True, seed=14, edit=drop)


@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_bwd_tau(gsa, torch, tau):
    _check(gsa, torch, 1, 2, 100, 64, 32, "f32", init=True, final=True, tau=tau, seed=9)


def _extreme(inp):
    x = inp["g"].f64.copy()
    x[..., 3, :] = -np.inf          # reset: alpha = 0
    x[..., 70:75, 2] = np.inf       # frozen slot: alpha = 1, nothing written
    x[..., 100, :5] = -30.0
    x[..., 130:140, 7] = 30.0
    x[..., 200:260, 1] = -np.inf
    inp["g"] = synth.stored(x, inp["g"].dtype)


@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64)])
def test_bwd_extreme_gates(gsa, torch, dtype, d, m):
    """Gates at +-inf and +-30: resets, frozen slots and near-saturated
    decays inside and across chunks."""
    _check(gsa, torch, 1, 2, 300, d, m, dtype, init=True, final=True, seed=13, edit=_extreme)


def test_bwd_empty_sequence(gsa, torch):
    """T = 0: the initial-state gradients are the final-state gradients."""
    B, H, d, m = 2, 3, 128, 64
    gi = synth.gsa_grad_inputs(B, H, 1, d, d, m, dtype="bf16", seed=3, final_std=1.0)
    empty = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    ge = torch.empty((B, H, 0, m), dtype=torch.bfloat16, device="cuda")
    dkf, dvf = to_dev(gi["dkf"], torch), to_dev(gi["dvf"], torch)
    out = gsa.gsa_bwd(empty, empty, empty, ge, empty, None, None, dkf, dvf, state_grads=True)
    torch.cuda.synchronize()
    assert torch.equal(out[4], dkf) and torch.equal(out[5], dvf)


def test_bwd_matches_chunkwise_forward_outputs(gsa, torch):
    """The backward recomputes the forward from chunk states of its own; the
    gradient of <dO, o> along q must equal what the forward kernels give by a
    central difference in float32 (a check independent of the oracle's
    backward)."""
    B, H, T, d, m = 1, 2, 200, 64, 32
    inp = synth.gsa_inputs(B, H, T, d, d, m, dtype="f32", seed=17, init_std=0.1)
    gi = synth.gsa_grad_inputs(B, H, T, d, d, m, dtype="f32", seed=18)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    do = to_dev(gi["do"], torch)
    dq = gsa.gsa_bwd(dev["q"], dev["k"], dev["v"], dev["g"], do, dev["k0"], dev["v0"])[0]
    u = torch.randn(dev["q"].shape, generator=torch.Generator(device="cuda").manual_seed(1),
                    device="cuda")
    eps = 1e-2

    def L(qx):
        o = gsa.gsa_fwd(qx, dev["k"], dev["v"], dev["g"], dev["k0"], dev["v0"])[0]
        return float((o.double() * do.double()).sum())
    num = (L(dev["q"] + eps * u) - L(dev["q"] - eps * u)) / (2 * eps)
    ana = float((dq.double() * u.double()).sum())
    print("directional dq: %.6e vs %.6e" % (ana, num))
    assert abs(ana - num) <= 5e-3 * abs(num)


@pytest.mark.parametrize("name", ["gsa_bf16_train_T2048", "gsa_bf16_train_T2048_rapid_forget",
                                  "gsa_bf16_train_T2048_extreme_forget"])
def test_bwd_training_shape_sampled(gsa, torch, name):
    """The training-shape workload (B8 H4 T2048 d128 m64, bf16) in the launch
    configuration the benchmark times, with its fast-forgetting variants (8
    slots at logits N(-10, 1): sub-chunk form; N(-40, 1): exact walks); five
    units against the oracle."""
    w = synth.WORKLOADS[name]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"], fast_slots=w.get("fast_slots", 0),
                           fast_shift=w.get("fast_shift", 0.0))
    gi = synth.gsa_grad_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                               seed=1)
    got = _run(gsa, torch, inp, gi, w["tau"])
    units = [0, 7, 13, 22, w["B"] * w["H"] - 1]
    _compare(got, _ref(inp, gi, w["tau"], units), "bf16", name + " sampled", units)


def test_bwd_long_context_sampled(gsa, torch):
    """The long-context shape (B1 H8 T16384, 256 chunks per unit) with initial
    states and final-state gradients; two units against the oracle."""
    w = synth.WORKLOADS["gsa_bf16_long_T16384"]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"])
    gi = synth.gsa_grad_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                               seed=2, final_std=1.0)
    got = _run(gsa, torch, inp, gi, w["tau"])
    units = [0, w["B"] * w["H"] - 1]
    _compare(got, _ref(inp, gi, w["tau"], units), "bf16", "B1 H8 T16384 sampled", units)


ELEMENTWISE = ["identity", "swish", "relu", "relu2"]


@pytest.mark.parametrize("nl", ELEMENTWISE)
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64)])
def test_bwd_elementwise_reads(gsa, torch, nl, dtype, d, m):
    """The backward of the forward with each element-wise read of Table 2."""
    _check(gsa, torch, 2, 2, 130, d, m, dtype, init=True, final=True, seed=60, nl=nl)


@pytest.mark.parametrize("nl", ["swish", "relu2"])
def test_bwd_elementwise_reads_extreme_gates(gsa, torch, nl):
    _check(gsa, torch, 1, 2, 300, 128, 64, "bf16", init=True, final=True, seed=61, edit=_extreme,
           nl=nl)


def test_bwd_elementwise_read_training_shape_sampled(gsa, torch):
    w = synth.WORKLOADS["gsa_bf16_train_T2048"]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"])
    gi = synth.gsa_grad_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                               seed=3)
    got = _run(gsa, torch, inp, gi, w["tau"], "swish")
    units = [3, w["B"] * w["H"] - 2]
    _compare(got, _ref(inp, gi, w["tau"], units, "swish"), "bf16", "B8 H4 T2048 swish sampled", units)


def test_bwd_event_hooks_and_repeatability(gsa, torch):
    """The dispatch-stamped launches give the plain launches' bits; a second
    call on a reused (dirty) workspace gives the same bits; the stamps of the
    two token walks are ordered."""
    from tests.test_gpu_parity import _hip_events
    inp = synth.gsa_inputs(2, 2, 300, 128, 128, 64, dtype="bf16", seed=70, init_std=0.1)
    gi = synth.gsa_grad_inputs(2, 2, 300, 128, 128, 64, dtype="bf16", seed=71, final_std=1.0)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {n: to_dev(gi[n], torch) for n in ("do", "dkf", "dvf")}
    ws = torch.empty(gsa.gsa_bwd_workspace_bytes(2, 2, 300, 128, 128, 64), dtype=torch.uint8,
                     device="cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"], dev["k0"], dev["v0"], ddev["dkf"],
            ddev["dvf"])
    a = gsa.gsa_bwd(*args, state_grads=True, workspace=ws)
    evs, ms, free = _hip_events(4)
    b = gsa.gsa_bwd(*args, state_grads=True, workspace=ws, events=evs)
    torch.cuda.synchronize()
    t = [ms(evs[0], evs[1]), ms(evs[2], evs[3]), ms(evs[0], evs[3])]
    free()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert t[0] > 0 and t[1] > 0 and t[2] >= t[0] + t[1], t


def test_autograd_function(gsa, torch):
    """gsa_autograd: torch.autograd through gsa_fwd / gsa_bwd gives the direct
    backward's bits and the oracle's gradients, for a loss on o and on the
    final states."""
    inp = synth.gsa_inputs(2, 2, 130, 128, 128, 64, dtype="bf16", seed=75, init_std=0.1)
    gi = synth.gsa_grad_inputs(2, 2, 130, 128, 128, 64, dtype="bf16", seed=76, final_std=1.0)
    leaves = {n: to_dev(inp[n], torch).requires_grad_(True) for n in ("q", "k", "v", "g", "k0", "v0")}
    W, A, Bv = (to_dev(gi[n], torch) for n in ("do", "dkf", "dvf"))
    o, kf, vf = gsa.gsa_autograd(*(leaves[n] for n in ("q", "k", "v", "g", "k0", "v0")), tau=8.0)
    loss = (o.float() * W.float()).sum() + (kf * A).sum() + (vf * Bv).sum()
    loss.backward()
    torch.cuda.synchronize()
    direct = gsa.gsa_bwd(*(leaves[n].detach() for n in ("q", "k", "v", "g")), W,
                         leaves["k0"].detach(), leaves["v0"].detach(), A, Bv, state_grads=True)
    for n, d in zip(("q", "k", "v", "g", "k0", "v0"), direct):
        assert torch.equal(leaves[n].grad, d), n
    ref = _ref(inp, gi, 8.0)
    _compare(dict(zip(GRADS, (leaves[n].grad for n in ("q", "k", "v", "g", "k0", "v0")))), ref,
             "bf16", "autograd B2 H2 T130")


@pytest.mark.parametrize("nl", ["softmax", "relu2"])
def test_autograd_function_without_states(gsa, torch, nl):
    """No initial states and a loss on o only (the final-state gradients
    arrive as None), with the softmax read and an element-wise one."""
    inp = synth.gsa_inputs(1, 3, 100, 64, 64, 32, dtype="f32", seed=77)
    gi = synth.gsa_grad_inputs(1, 3, 100, 64, 64, 32, dtype="f32", seed=78)
    leaves = {n: to_dev(inp[n], torch).requires_grad_(True) for n in "qkvg"}
    W = to_dev(gi["do"], torch)
    o, _, _ = gsa.gsa_autograd(*(leaves[n] for n in "qkvg"), tau=8.0, nonlinearity=nl)
    (o * W).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.gsa_bwd(*(inp[n].f64 for n in "qkvg"), gi["do"].f64, tau=8.0, nonlinearity=nl)
    errs = {n: rel_err(to_np(leaves[n].grad), ref["d" + n]) for n in "qkvg"}
    print("autograd %s no states: %s" % (nl, errs))
    assert max(errs.values()) <= TOL["f32"], errs


def test_autograd_double_backward_raises(gsa, torch):
    """The backward is not itself differentiable: asking for a gradient of a
    gradient raises instead of silently dropping the second-order terms."""
    inp = synth.gsa_inputs(1, 1, 40, 64, 64, 32, dtype="f32", seed=79)
    leaves = {n: to_dev(inp[n], torch).requires_grad_(True) for n in "qkvg"}
    o, _, _ = gsa.gsa_autograd(*(leaves[n] for n in "qkvg"), tau=8.0)
    (gq,) = torch.autograd.grad(o.sum(), leaves["q"], create_graph=True)
    with pytest.raises(RuntimeError):
        torch.autograd.grad(gq.sum(), leaves["k"])


def test_bwd_exact_chunks_inside_segments_sampled(gsa, torch):
    """Segments of several chunks where every chunk leaves the chunk form's
    range (8 of 64 slots at logits N(-10, 1), 64-token decay products near
    2^-115: the sub-chunk form) and one chunk in the middle of a segment
    holds gates at +-inf (an exact walk): the state, the reverse map, the
    adjoint and the gate sums carry across sub-chunk-form and exact chunks
    alike.  Sampled units against the oracle."""
    B, H, T = 8, 4, 1024  # 32 units of 16 chunks: segments of 2 chunks
    inp = synth.gsa_inputs(B, H, T, 128, 128, 64, dtype="bf16", seed=81, init_std=0.1, fast_slots=8,
                           fast_shift=-10.0)
    x = inp["g"].f64.copy()
    x[:, :, 70:90, 20:30] = np.inf
    x[:, :, 75, 40:] = -np.inf
    inp["g"] = synth.stored(x, "bf16")
    gi = synth.gsa_grad_inputs(B, H, T, 128, 128, 64, dtype="bf16", seed=82, final_std=1.0)
    got = _run(gsa, torch, inp, gi, 8.0)
    units = [0, 13, 31]
    _compare(got, _ref(inp, gi, 8.0, units=units), "bf16", "exact chunks inside segments", units=units)


@pytest.mark.parametrize("mean", [-7.3, -8.0])
def test_bwd_decay_near_the_floor(gsa, torch, mean):
    """Gate logits N(mean, 0.05): 64-token decay products ~2^-84 (factorised
    with X up to ~2^84) and ~2^-92 (around the 2^-90 floor: chunks of both
    forms), through the forward and reverse sweeps."""
    def mut(inp):
        r = np.random.default_rng(6)
        inp["g"] = synth.stored(mean + 0.05 * r.standard_normal(inp["g"].shape), "bf16")
    _check(gsa, torch, 2, 2, 64 * 5 + 11, 128, 64, "bf16", init=True, final=True, seed=83, edit=mut)


@pytest.mark.parametrize("case", ["fast_slots", "sub_floor", "per_chunk"])
@pytest.mark.parametrize("d,m", [(128, 64), (64, 32), (128, 32), (64, 64)])
def test_bwd_subchunk_form(gsa, torch, case, d, m):
    """Chunks out of the chunk form's range run both sweeps with 16-token
    sub-chunk reference points: 8 slots at g ~ N(-10, 1) everywhere
    ("fast_slots"), 8 slots at g ~ N(-30.5, 0.05) everywhere (16-token
    products ~2^-88, X up to ~2^88: "sub_floor"), and the chunk / sub-chunk
    / exact regimes in turn ("per_chunk"); initial states and final-state
    gradients on.  (With every slot near that floor all slot scores of a
    token are nearly equal and dz = s (ds - s.ds) cancels to a few percent of
    its terms, which bf16 operands do not resolve to this bar.)"""
    edit = {"fast_slots": gates_fast_slots(8, -10.0), "sub_floor": gates_fast_slots(8, -30.5, 0.05),
            "per_chunk": gates_regime_per_chunk}[case]
    _check(gsa, torch, 2, 2, 64 * 5 + 11, d, m, "bf16", init=True, final=True, seed=84, edit=edit)


@pytest.mark.parametrize("nl", ["identity", "swish", "relu2"])
def test_bwd_subchunk_form_elementwise_reads(gsa, torch, nl):
    _check(gsa, torch, 1, 2, 64 * 4 + 9, 128, 64, "bf16", init=True, final=True, seed=85,
           edit=gates_fast_slots(8, -10.0), nl=nl)
