"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded stored inputs.

Bar (max |x - y| / max |y| per output tensor): 1e-4 for float32 inputs,
2e-2 for bfloat16 inputs with float32 state and accumulation.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (TOL, gates_fast_slots, gates_normal, gates_regime_per_chunk, rel_err, to_dev,
                                to_np)

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


def _run_gsa(gsa, torch, inp, tau, final=True, cps=0):
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, k0, v0, tau=tau, final_state=final, chunks_per_segment=cps)
    torch.cuda.synchronize()
    return o, kf, vf


def _oracle_gsa(inp, tau, units=None):
    f = lambda x: None if x is None else (x.f64 if units is None else x.f64.reshape(-1, *x.shape[2:])[units][:, None])
    return oracle.gsa_fwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]), f(inp["k0"]),
                          f(inp["v0"]), tau=tau, nthreads=oracle.max_threads())


def _check_gsa(gsa, torch, B, H, T, d, m, dtype, init=False, tau=8.0, cps=0, g_shift=0.0,
               seed=0, mutate=None):
    inp = synth.gsa_inputs(B, H, T, d, d, m, dtype=dtype, seed=seed, g_shift=g_shift,
                           init_std=0.1 if init else None)
    if mutate is not None:
        mutate(inp)
    o, kf, vf = _run_gsa(gsa, torch, inp, tau, final=True, cps=cps)
    ref = _oracle_gsa(inp, tau)
    tol = TOL[dtype]
    eo, ek, ev = rel_err(to_np(o), ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"])
    print("gsa B%d H%d T%d d%d m%d %s init=%s cps=%d: o %.2e kf %.2e vf %.2e" %
          (B, H, T, d, m, dtype, init, cps, eo, ek, ev))
    assert eo <= tol and ek <= tol and ev <= tol
    return o


# ----------------------------------------------------------------- GSA
def test_gsa_f32_small_workload(gsa, torch):
    """B1 H2 T256 d64 m32, float32, zero state, seed 0 (q,k,v scaled 1/8)."""
    w = synth.WORKLOADS["gsa_f32_small"]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype="f32",
                           seed=0, qkv_scale=w["qkv_scale"])
    o, kf, vf = _run_gsa(gsa, torch, inp, w["tau"])
    ref = _oracle_gsa(inp, w["tau"])
    for x, y in ((o, ref["o"]), (kf, ref["kf"]), (vf, ref["vf"])):
        assert rel_err(to_np(x), y) <= 1e-4


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200, 320])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("f32", 64, 16), ("bf16", 128, 64),
                                       ("bf16", 64, 32), ("bf16", 128, 32), ("f32", 128, 16),
                                       ("bf16", 64, 64)])
def test_gsa_shapes(gsa, torch, T, dtype, d, m):
    _check_gsa(gsa, torch, 2, 2, T, d, m, dtype, init=(T % 2 == 1), seed=T)


@pytest.mark.parametrize("which", ["k0", "v0"])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 128, 128)])
def test_gsa_one_initial_state(gsa, torch, which, dtype, d, m):
    """Only one of the two initial slot states given (the other zero), across
    several segments: each start state is loaded on its own."""
    def drop(inp):
        inp["v0" if which == "k0" else "k0"] = None
    _check_gsa(gsa, torch, 2, 2, 64 * 5 + 7, d, m, dtype, init=True, cps=2, seed=13, mutate=drop)


@pytest.mark.parametrize("tau", [1.0, 2.0, 32.0, 256.0])
@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 64, 32)])
def test_gsa_tau(gsa, torch, tau, dtype, d, m):
    """The damping exponent 1/tau of the forget gate (Sec. 3.3) away from 8:
    tau = 1 and 2 decay fast (sub-chunk reference points and exact chunks
    among the logits N(0, 1)), tau = 32 and 256 keep 1 - alpha small, where
    the telescoped factors difference nearly equal terms."""
    _check_gsa(gsa, torch, 2, 2, 64 * 4 + 21, d, m, dtype, init=True, tau=tau, seed=11, cps=2)


@pytest.mark.parametrize("cps", [1, 2, 3, 100])
def test_gsa_segmentations(gsa, torch, cps):
    """The chunk-state scan must give the same result for any segment split."""
    _check_gsa(gsa, torch, 1, 3, 64 * 7 + 5, 128, 64, "bf16", init=True, cps=cps, seed=3)
    _check_gsa(gsa, torch, 1, 2, 64 * 5 + 9, 64, 32, "f32", init=True, cps=cps, seed=4)


@pytest.mark.parametrize("cps", [1, 2, 3, 4])
def test_gsa_bf16_segments_xcd_placement(gsa, torch, cps):
    """8 units, so every segment of a unit runs on one XCD; 10 chunks with a
    ragged tail and initial states.  cps 4 / 3: 3 / 4 segments, whose output
    workgroups build their start states from 2 / 3 segment maps themselves;
    cps 2 / 1: 5 / 10 segments, start states from the scan kernel."""
    _check_gsa(gsa, torch, 2, 4, 64 * 9 + 13, 128, 64, "bf16", init=True, cps=cps, seed=31)


def _extreme(inp):
    g = inp["g"]
    x = g.f64.copy()
    x[..., 3, :] = -np.inf
    x[..., 70:75, 2] = np.inf
    x[..., 100, :5] = -30.0
    x[..., 130:140, 7] = 30.0
    x[..., 200:260, 1] = -np.inf
    inp["g"] = synth.stored(x, g.dtype)


@pytest.mark.parametrize("dtype,d,m", [("f32", 64, 32), ("bf16", 128, 64)])
def test_gsa_extreme_gates(gsa, torch, dtype, d, m):
    """alpha = 0 / alpha = 1 tokens (g = -inf / +inf, +-30): chunks whose decay
    product falls below the factorised form's floor (e^-40 in float32; in
    bfloat16 2^-90 over a 16-token sub-chunk) take the exact token
    recurrence."""
    for cps in (0, 1):
        _check_gsa(gsa, torch, 1, 2, 300, d, m, dtype, init=True, cps=cps, mutate=_extreme, seed=7)


def test_gsa_split_handoff_and_inplace(gsa, torch):
    """fwd over [0,T1) then [T1,T) from the handed-off state == fwd over [0,T);
    the second call advances the state in place (k_final is k0)."""
    inp = synth.gsa_inputs(2, 2, 333, 64, 64, 32, dtype="f32", seed=11, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    o_full, kf, vf = gsa.gsa_fwd(q, k, v, g, k0, v0, final_state=True, chunks_per_segment=1)
    T1 = 130
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, k1, v1 = gsa.gsa_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1), k0, v0,
                             final_state=True)
    o2, k2, v2 = gsa.gsa_fwd(sl(q, T1, 333), sl(k, T1, 333), sl(v, T1, 333), sl(g, T1, 333), k1, v1,
                             final_state=True, k_final=k1, v_final=v1, chunks_per_segment=1)
    torch.cuda.synchronize()
    assert k2.data_ptr() == k1.data_ptr()
    full = to_np(o_full)
    assert rel_err(np.concatenate([to_np(o1), to_np(o2)], axis=2), full) <= 1e-5
    assert rel_err(to_np(k2), to_np(kf)) <= 1e-5 and rel_err(to_np(v2), to_np(vf)) <= 1e-5


def test_gsa_empty_and_tiny(gsa, torch):
    inp = synth.gsa_inputs(1, 2, 0, 64, 64, 32, dtype="f32", seed=1, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, k0, v0, final_state=True)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(to_np(kf), inp["k0"].f64) and np.array_equal(to_np(vf), inp["v0"].f64)
    o, _, _ = gsa.gsa_fwd(q[:0], k[:0], v[:0], g[:0])   # B = 0
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_gsa_deterministic(gsa, torch):
    inp = synth.gsa_inputs(2, 4, 700, 128, 128, 64, dtype="bf16", seed=5)
    a = _run_gsa(gsa, torch, inp, 8.0)[0]
    b = _run_gsa(gsa, torch, inp, 8.0)[0]
    assert torch.equal(a, b)


# ----------------------------------------------------------------- GLA
def _check_gla(gsa, torch, B, H, T, d, dtype, init=False, tau=16.0, cps=0, seed=0, mutate=None):
    inp = synth.gla_inputs(B, H, T, d, d, dtype=dtype, seed=seed, init_std=0.1 if init else None)
    if mutate is not None:
        mutate(inp)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o, sf = gsa.gla_fwd(q, k, v, g, to_dev(inp["s0"], torch), tau=tau, final_state=True,
                        chunks_per_segment=cps)
    torch.cuda.synchronize()
    s0 = None if inp["s0"] is None else inp["s0"].f64
    ref = oracle.gla_fwd(inp["q"].f64, inp["k"].f64, inp["v"].f64, inp["g"].f64, s0, tau=tau,
                         nthreads=oracle.max_threads())
    eo, es = rel_err(to_np(o), ref["o"]), rel_err(to_np(sf), ref["sf"])
    print("gla B%d H%d T%d d%d %s cps=%d: o %.2e sf %.2e" % (B, H, T, d, dtype, cps, eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("T", [1, 50, 64, 129, 300])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_gla_shapes(gsa, torch, T, dtype, d):
    _check_gla(gsa, torch, 2, 2, T, d, dtype, init=(T % 2 == 0), seed=T)


@pytest.mark.parametrize("tau", [1.0, 4.0, 64.0])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_gla_tau(gsa, torch, tau, dtype, d):
    """GLA's gate damping 1/tau away from the workload's 16."""
    _check_gla(gsa, torch, 2, 2, 64 * 4 + 21, d, dtype, init=True, tau=tau, cps=2, seed=12)


@pytest.mark.parametrize("cps", [1, 3])
def test_gla_segmentations(gsa, torch, cps):
    _check_gla(gsa, torch, 1, 2, 64 * 6 + 3, 128, "bf16", init=True, cps=cps, seed=2)


def test_gla_state_split_with_empty_subsegment(gsa, torch):
    # 64 units, 10 chunks, 5 per output segment: the bf16 state-map pass splits
    # each segment into 4 sub-segments of 2 chunks, the last of them empty
    _check_gla(gsa, torch, 8, 8, 640, 64, "bf16", init=True, cps=5, seed=4)


@pytest.mark.parametrize("cps", [2, 7])
def test_gla_bf16_split_ragged(gsa, torch, cps):
    # few units: sub-segments of one chunk; ragged tail
    _check_gla(gsa, torch, 1, 3, 64 * 9 + 17, 128, "bf16", init=True, cps=cps, seed=11)


@pytest.mark.parametrize("cps", [1, 2, 3])
def test_gla_bf16_folded_start_states(gsa, torch, cps):
    """8 units, 4 chunks with a ragged tail, initial state.  cps 1: 4 segments
    of one chunk (3 maps before the last); cps 2 / 3: 2 segments whose state
    maps split into 2 / 3 sub-segments.  Few enough maps that the output
    workgroups fold them into their start states themselves."""
    _check_gla(gsa, torch, 2, 4, 64 * 3 + 17, 128, "bf16", init=True, cps=cps, seed=41)


def test_gla_extreme_gates(gsa, torch):
    def mut(inp):
        x = inp["g"].f64.copy()
        x[..., 10, :] = -np.inf
        x[..., 80:90, 5] = np.inf
        x[..., 150:220, 3] = -np.inf
        inp["g"] = synth.stored(x, inp["g"].dtype)
    _check_gla(gsa, torch, 1, 2, 260, 64, "f32", init=True, mutate=mut, seed=9)
    _check_gla(gsa, torch, 1, 2, 260, 128, "bf16", init=True, mutate=mut, seed=9, cps=1)
    _check_gla(gsa, torch, 1, 2, 260, 64, "bf16", init=True, mutate=mut, seed=9, cps=2)
    _check_gla(gsa, torch, 1, 2, 260, 128, "bf16", init=True, mutate=mut, seed=9)


# -------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32), ("f32", 128, 64),
                                       ("bf16", 64, 32), ("f32", 64, 16)])
def test_decode_step(gsa, torch, dtype, d, m):
    inp = synth.decode_inputs(3, 5, d, d, m, dtype=dtype, seed=m)
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs)
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(inp["q"].f64, inp["k"].f64, inp["v"].f64, inp["g"].f64,
                                        inp["kstate"].f64, inp["vstate"].f64)
    tol = TOL[dtype]
    assert rel_err(to_np(o), ro) <= tol
    assert rel_err(to_np(ks), rk) <= 1e-5 and rel_err(to_np(vs), rv) <= 1e-5


@pytest.mark.parametrize("tau", [1.0, 64.0])
@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32)])
def test_decode_step_tau(gsa, torch, tau, dtype, d, m):
    """The decode step's gate damping 1/tau away from 8."""
    inp = synth.decode_inputs(3, 5, d, d, m, dtype=dtype, seed=m + 7)
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs, tau=tau)
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(inp["q"].f64, inp["k"].f64, inp["v"].f64, inp["g"].f64,
                                        inp["kstate"].f64, inp["vstate"].f64, tau=tau)
    assert rel_err(to_np(o), ro) <= TOL[dtype]
    assert rel_err(to_np(ks), rk) <= 1e-5 and rel_err(to_np(vs), rv) <= 1e-5


def test_decode_chain_equals_fwd(gsa, torch):
    """T chained decode steps reproduce the chunkwise forward (float32)."""
    inp = synth.gsa_inputs(2, 2, 70, 64, 64, 32, dtype="f32", seed=21, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    ks, vs = to_dev(inp["k0"], torch).clone(), to_dev(inp["v0"], torch).clone()
    o_fwd, kf, vf = gsa.gsa_fwd(q, k, v, g, to_dev(inp["k0"], torch), to_dev(inp["v0"], torch),
                                final_state=True)
    outs = []
    for t in range(70):
        outs.append(gsa.gsa_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                        v[:, :, t].contiguous(), g[:, :, t].contiguous(), ks, vs))
    torch.cuda.synchronize()
    assert rel_err(np.stack([to_np(x) for x in outs], axis=2), to_np(o_fwd)) <= 1e-5
    assert rel_err(to_np(ks), to_np(kf)) <= 1e-5 and rel_err(to_np(vs), to_np(vf)) <= 1e-5


# ------------------------------------------------------------ timing hooks
def _hip_events(n):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)

    def ms(a, b):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return f.value

    def free():
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    return evs, ms, free


@pytest.mark.parametrize("dtype,cps", [("bf16", 2), ("bf16", 64), ("f32", 2)])
def test_event_hooks_give_identical_results(gsa, torch, dtype, cps):
    """The timed launches (dispatch-stamped events) compute exactly what the
    plain ones do, and the stamps are ordered."""
    inp = synth.gsa_inputs(2, 2, 300, 64, 64, 32, dtype=dtype, seed=7)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o1, _, _ = gsa.gsa_fwd(q, k, v, g, tau=8.0, final_state=False, chunks_per_segment=cps)
    evs, ms, free = _hip_events(4)
    o2, _, _ = gsa.gsa_fwd(q, k, v, g, tau=8.0, final_state=False, chunks_per_segment=cps,
                           events=evs)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    t = [ms(evs[0], evs[1]), ms(evs[1], evs[2]), ms(evs[2], evs[3]), ms(evs[0], evs[3])]
    free()
    assert t[2] > 0 and t[3] >= t[2] and min(t[0], t[1]) >= 0, t


def test_decode_event_hooks(gsa, torch):
    inp = synth.decode_inputs(8, 2, 128, 128, 64, dtype="bf16", seed=3)
    tok = {n: to_dev(inp[n], torch) for n in "qkvg"}
    ks1, vs1 = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    ks2, vs2 = ks1.clone(), vs1.clone()
    o1 = gsa.gsa_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], ks1, vs1, tau=8.0)
    evs, ms, free = _hip_events(2)
    o2 = gsa.gsa_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], ks2, vs2, tau=8.0, events=evs)
    torch.cuda.synchronize()
    t = ms(evs[0], evs[1])
    free()
    assert torch.equal(o1, o2) and torch.equal(ks1, ks2) and torch.equal(vs1, vs2)
    assert t > 0


# ------------------------------------------------- decay regimes, hand-offs
def _decay_chunks(chunks, value):
    """Gate logit `value` on every token of the listed 64-token chunks."""
    def mut(inp):
        x = inp["g"].f64.copy()
        for c in chunks:
            x[..., 64 * c:64 * c + 64, :] = value
        inp["g"] = synth.stored(x, inp["g"].dtype)
    return mut


def _shift_gates(shift):
    def mut(inp):
        inp["g"] = synth.stored(inp["g"].f64 + shift, inp["g"].dtype)
    return mut


@pytest.mark.parametrize("case", ["all", "mixed", "near_floor"])
def test_gsa_bf16_strong_decay(gsa, torch, case):
    # alpha = sigmoid(g)^(1/8).  "all": g ~ N(-8, 1) makes the 64-token decay
    # products ~2^-92, around the 2^-90 floor of the chunk form, so chunks
    # take either the chunk form or the sub-chunk form.  "mixed": g = -12 on
    # chunks 1 and 3 (64-token products ~2^-138, 16-token ~2^-35: sub-chunk
    # form) and N(0, 1) elsewhere.  "near_floor": g ~ N(-7.3, 0.05), products
    # ~2^-84: every chunk in the chunk form with X up to ~2^84.
    mut = {"all": _shift_gates(-8.0), "mixed": _decay_chunks((1, 3), -12.0),
           "near_floor": gates_normal(-7.3, 0.05)}[case]
    for cps in (0, 1):
        _check_gsa(gsa, torch, 2, 2, 64 * 5 + 11, 128, 64, "bf16", init=True, cps=cps, seed=21, mutate=mut)


@pytest.mark.parametrize("case", ["fast_slots", "sub_floor", "per_chunk"])
@pytest.mark.parametrize("d,m", [(128, 64), (128, 32), (64, 64), (64, 32)])
def test_gsa_bf16_subchunk_form(gsa, torch, case, d, m):
    """Chunks whose 64-token decay product falls below the chunk form's 2^-90
    floor in some slot run with 16-token sub-chunk reference points, and only
    a sub-chunk product below 2^-90 sends a chunk to the exact walk.
    "fast_slots": 8 slots at g ~ N(-10, 1) on every token (64-token products
    ~2^-115, every chunk in the sub-chunk form).  "sub_floor": every slot at
    g ~ N(-30.5, 0.05) (16-token products ~2^-88: X up to ~2^88).
    "per_chunk": the plain, sub-chunk and exact regimes in turn."""
    mut = {"fast_slots": gates_fast_slots(8, -10.0), "sub_floor": gates_normal(-30.5, 0.05),
           "per_chunk": gates_regime_per_chunk}[case]
    for cps in (0, 1):
        _check_gsa(gsa, torch, 2, 2, 64 * 5 + 11, d, m, "bf16", init=True, cps=cps, seed=23, mutate=mut)


@pytest.mark.parametrize("case", ["all", "mixed", "near_floor"])
def test_gla_bf16_strong_decay(gsa, torch, case):
    # tau = 16: g ~ N(-12, 1) makes every 64-token product ~2^-70 (factorised
    # near the floor); "mixed": g = -12 on chunks 1 and 3 only; "near_floor":
    # g ~ N(-15.5, 0.05), products ~2^-89
    mut = {"all": _shift_gates(-12.0), "mixed": _decay_chunks((1, 3), -12.0),
           "near_floor": gates_normal(-15.5, 0.05)}[case]
    for cps in (0, 1):
        _check_gla(gsa, torch, 1, 3, 64 * 5 + 11, 128, "bf16", init=True, cps=cps, seed=22, mutate=mut)


def test_gsa_bf16_split_handoff(gsa, torch):
    """bf16: fwd over [0,T1) then [T1,T) from the handed-off fp32 state agrees
    with one call over [0,T) and with the oracle."""
    inp = synth.gsa_inputs(2, 2, 64 * 6 + 7, 128, 128, 64, dtype="bf16", seed=23, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    T, T1 = q.shape[2], 64 * 2 + 30
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, k1, v1 = gsa.gsa_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1), k0, v0,
                             final_state=True)
    # the second call advances the state in place (4 chunks, one per segment)
    o2, k2, v2 = gsa.gsa_fwd(sl(q, T1, T), sl(k, T1, T), sl(v, T1, T), sl(g, T1, T), k1, v1,
                             final_state=True, k_final=k1, v_final=v1, chunks_per_segment=1)
    torch.cuda.synchronize()
    assert k2.data_ptr() == k1.data_ptr() and v2.data_ptr() == v1.data_ptr()
    ref = _oracle_gsa(inp, 8.0)
    o = np.concatenate([to_np(o1), to_np(o2)], axis=2)
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(to_np(k2), ref["kf"]) <= TOL["bf16"] and rel_err(to_np(v2), ref["vf"]) <= TOL["bf16"]


def test_gla_bf16_split_handoff_empty_and_deterministic(gsa, torch):
    inp = synth.gla_inputs(1, 2, 64 * 5 + 3, 128, 128, dtype="bf16", seed=24, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    s0 = to_dev(inp["s0"], torch)
    T, T1 = q.shape[2], 64 + 17
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, s1 = gsa.gla_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1), s0, final_state=True)
    # the second call advances the state in place (4 chunks, one per segment)
    o2, s2 = gsa.gla_fwd(sl(q, T1, T), sl(k, T1, T), sl(v, T1, T), sl(g, T1, T), s1, final_state=True,
                         s_final=s1, chunks_per_segment=1)
    oa, _ = gsa.gla_fwd(q, k, v, g, s0)
    ob, _ = gsa.gla_fwd(q, k, v, g, s0)
    # T = 0: the final state is the initial one
    oz, sz = gsa.gla_fwd(sl(q, 0, 0), sl(k, 0, 0), sl(v, 0, 0), sl(g, 0, 0), s0, final_state=True)
    torch.cuda.synchronize()
    ref = oracle.gla_fwd(inp["q"].f64, inp["k"].f64, inp["v"].f64, inp["g"].f64, inp["s0"].f64,
                         tau=16.0, nthreads=oracle.max_threads())
    assert rel_err(np.concatenate([to_np(o1), to_np(o2)], axis=2), ref["o"]) <= TOL["bf16"]
    assert s2.data_ptr() == s1.data_ptr() and rel_err(to_np(s2), ref["sf"]) <= TOL["bf16"]
    assert torch.equal(oa, ob)
    assert oz.numel() == 0 and np.array_equal(to_np(sz), inp["s0"].f64)
