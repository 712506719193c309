"""GPU parity of the packed variable-length GSA forward (gsa_fwd_varlen) and of
the serving chain it feeds: prefill a batch of prompts of different lengths in
one call, then advance every (sequence, head) unit with gsa_decode_step from
the prefill's final states.

Each sequence is an independent run of the method, so the oracle is the plain
recurrence on each sequence's own slice (and, for the chain, on the prompt
followed by the decoded tokens).  Bar: max |x - y| / max |y| <= 2e-2 per output
tensor (bf16 inputs, fp32 state).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, RawEvents, gates_fast_slots, rel_err, to_dev, to_np

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


def _seq(x, cu, s):
    """Sequence s of a packed head-major [H, total, d] array -> [1, H, T_s, d]."""
    return x[:, cu[s]:cu[s + 1]][None]


def _oracle_each(inp, tau=8.0):
    """The oracle on every sequence separately: (o [H,total,dv], kf, vf [n,H,m,d])."""
    cu = inp["cu_seqlens"]
    n = len(cu) - 1
    H, total, dv = inp["v"].shape
    m, dk = inp["g"].shape[-1], inp["q"].shape[-1]
    o = np.zeros((H, total, dv))
    kf = np.zeros((n, H, m, dk))
    vf = np.zeros((n, H, m, dv))
    for s in range(n):
        k0 = None if inp["k0"] is None else inp["k0"].f64[s:s + 1]
        v0 = None if inp["v0"] is None else inp["v0"].f64[s:s + 1]
        r = oracle.gsa_fwd(*(_seq(inp[x].f64, cu, s) for x in "qkvg"), k0, v0, tau=tau,
                           nthreads=oracle.max_threads())
        o[:, cu[s]:cu[s + 1]] = r["o"][0]
        kf[s], vf[s] = r["kf"][0], r["vf"][0]
    return o, kf, vf


def _run(gsa, torch, inp, cps=0, in_place=False):
    q, k, v, g = (to_dev(inp[x], torch) for x in "qkvg")
    k0, v0 = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    kw = dict(k_final=k0, v_final=v0) if in_place else {}
    o, kf, vf = gsa.gsa_fwd_varlen(q, k, v, g, inp["cu_seqlens"], k0, v0, final_state=True,
                                   chunks_per_segment=cps, **kw)
    torch.cuda.synchronize()
    if in_place:
        assert kf.data_ptr() == k0.data_ptr() and vf.data_ptr() == v0.data_ptr()
    return o, kf, vf


def _check(gsa, torch, lengths, H, d, m, init, cps=0, seed=0, in_place=False, edit=None):
    inp = synth.varlen_inputs(lengths, H, d, d, m, dtype="bf16", seed=seed,
                              init_std=0.1 if init else None)
    if edit is not None:
        edit(inp)
    o, kf, vf = _run(gsa, torch, inp, cps, in_place)
    ro, rk, rv = _oracle_each(inp)
    errs = [rel_err(to_np(o), ro) if ro.size else 0.0, rel_err(to_np(kf), rk), rel_err(to_np(vf), rv)]
    print("varlen lengths=%s H%d d%d m%d init=%s cps=%d: o %.2e kf %.2e vf %.2e"
          % (lengths, H, d, m, init, cps, *errs))
    assert max(errs) <= TOL["bf16"], errs
    if not init:
        empty = [s for s, L in enumerate(lengths) if L == 0]
        assert np.all(to_np(kf)[empty] == 0.0) and np.all(to_np(vf)[empty] == 0.0)


MIX = [0, 1, 63, 64, 65, 200, 1000, 130, 0, 7]


@pytest.mark.parametrize("cps", [0, 1, 2, 3, 100])
def test_varlen_mixed_lengths(gsa, torch, cps):
    """Empty, one-token, sub-chunk, exact-chunk, ragged and multi-segment
    sequences in one call, with initial states; every segment split (the
    scan, maps folded in the output kernel, one segment)."""
    _check(gsa, torch, MIX, 2, 128, 64, init=True, cps=cps, seed=cps + 1)


@pytest.mark.parametrize("cps", [0, 1])
def test_varlen_subchunk_form(gsa, torch, cps):
    """The packed batch with 8 slots at logits N(-10, 1) on every token
    (chunks in the 16-token sub-chunk form) and one slot at -inf for three
    tokens of the 1000-token sequence (an exact chunk)."""
    def edit(inp):
        gates_fast_slots(8, -10.0)(inp)
        x = inp["g"].f64.copy()
        t = int(inp["cu_seqlens"][6]) + 70
        x[:, t:t + 3, 20] = -np.inf
        inp["g"] = synth.stored(x, "bf16")
    _check(gsa, torch, MIX, 2, 128, 64, init=True, cps=cps, seed=cps + 11, edit=edit)


@pytest.mark.parametrize("d,m", [(128, 64), (64, 32), (128, 32), (64, 64)])
def test_varlen_shapes(gsa, torch, d, m):
    _check(gsa, torch, [300, 17, 0, 129], 3, d, m, init=False, seed=d + m)


def test_varlen_in_place_state_advance(gsa, torch):
    _check(gsa, torch, [500, 70, 0, 260], 2, 128, 64, init=True, cps=1, seed=5, in_place=True)


def test_varlen_all_empty_and_single(gsa, torch):
    _check(gsa, torch, [0, 0, 0], 2, 128, 64, init=True, seed=6)
    _check(gsa, torch, [777], 4, 128, 64, init=True, seed=7)


def test_varlen_all_empty_records_events(gsa, torch):
    """A call whose only group holds empty sequences still records its four
    timing hooks (a caller timing it needs every event recorded)."""
    ev = RawEvents()
    evs = ev.create(4)
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    eg = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k0 = torch.randn((3, 2, 64, 128), device="cuda")
    _, kf, _ = gsa.gsa_fwd_varlen(e, e, e, eg, [0, 0, 0, 0], k0, None, final_state=True, events=evs)
    torch.cuda.synchronize()
    assert torch.equal(kf, k0)
    for a, b in ((0, 1), (2, 3), (0, 3)):
        assert ev.elapsed(evs[a], evs[b]) >= 0.0


def test_varlen_equal_lengths_is_the_dense_call(gsa, torch):
    """Equal lengths: the packed call splits like the dense batch and gives
    the same bits (same kernels, same segments)."""
    B, H, T = 4, 4, 1000
    dense = synth.gsa_inputs(B, H, T, 128, 128, 64, dtype="bf16", seed=8, init_std=0.1)
    dev = {x: to_dev(dense[x], torch) for x in ("q", "k", "v", "g", "k0", "v0")}
    o_d, kf_d, vf_d = gsa.gsa_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["k0"], dev["v0"],
                                  final_state=True)
    pk = {x: dev[x].permute(1, 0, 2, 3).reshape(H, B * T, -1).contiguous() for x in "qkvg"}
    cu = [i * T for i in range(B + 1)]
    o_v, kf_v, vf_v = gsa.gsa_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], cu, dev["k0"],
                                         dev["v0"], final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o_v, o_d.permute(1, 0, 2, 3).reshape(H, B * T, -1))
    assert torch.equal(kf_v, kf_d) and torch.equal(vf_v, vf_d)


def test_prefill_then_decode(gsa, torch):
    """The serving chain: one packed prefill of prompts of different lengths,
    then three decode steps of every unit from its final states, against the
    oracle on each prompt followed by its decoded tokens."""
    lengths = [40, 0, 300, 64, 1, 129]
    n, H, d, m, steps = len(lengths), 2, 128, 64, 3
    inp = synth.varlen_inputs(lengths, H, d, d, m, dtype="bf16", seed=9, init_std=0.1)
    _, ks, vs = _run(gsa, torch, inp)
    toks = [synth.decode_inputs(n, H, d, d, m, dtype="bf16", seed=100 + i) for i in range(steps)]
    outs = []
    for tk in toks:
        outs.append(gsa.gsa_decode_step(*(to_dev(tk[x], torch) for x in "qkvg"), ks, vs))
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    worst = 0.0
    for s in range(n):
        cat = {x: np.concatenate([_seq(inp[x].f64, cu, s)] +
                                 [tk[x].f64[s:s + 1, :, None] for tk in toks], axis=2)
               for x in "qkvg"}
        r = oracle.gsa_fwd(cat["q"], cat["k"], cat["v"], cat["g"], inp["k0"].f64[s:s + 1],
                           inp["v0"].f64[s:s + 1], tau=8.0)
        for i in range(steps):
            worst = max(worst, rel_err(to_np(outs[i])[s], r["o"][0, :, lengths[s] + i]))
        worst = max(worst, rel_err(to_np(ks)[s], r["kf"][0]), rel_err(to_np(vs)[s], r["vf"][0]))
    print("prefill + %d decode steps: worst rel err %.2e" % (steps, worst))
    assert worst <= TOL["bf16"]


def test_serving_workload_sampled(gsa, torch):
    """The serving workload's prefill (256 prompts, H16, log-uniform lengths in
    [16, 1024]) in the launch configuration the benchmark times; a sample of
    sequences against the oracle."""
    w = synth.WORKLOADS["gsa_bf16_serve_N256"]
    lengths = synth.varlen_lengths(w["N"], w["len_lo"], w["len_hi"], seed=0)
    inp = synth.varlen_inputs(lengths, w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"], seed=0,
                              qkv_scale=w["qkv_scale"], g_shift=w["g_shift"])
    o, kf, vf = _run(gsa, torch, inp)
    cu = inp["cu_seqlens"]
    on, kn, vn = to_np(o), to_np(kf), to_np(vf)
    picks = [int(np.argmax(lengths)), int(np.argmin(lengths)), 0, 100, w["N"] - 1]
    worst = 0.0
    for s in picks:
        r = oracle.gsa_fwd(*(_seq(inp[x].f64, cu, s) for x in "qkvg"), tau=w["tau"],
                           nthreads=oracle.max_threads())
        worst = max(worst, rel_err(on[:, cu[s]:cu[s + 1]], r["o"][0]), rel_err(kn[s], r["kf"][0]),
                    rel_err(vn[s], r["vf"][0]))
    print("serving prefill sampled sequences %s: worst rel err %.2e" % (picks, worst))
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("cps", [0, 1])
def test_varlen_more_than_256_sequences(gsa, torch, cps):
    """600 sequences run as three groups of up to 256; the middle group holds
    only empty sequences (its final states are the initial ones)."""
    r = np.random.default_rng(31)
    lengths = list(r.integers(1, 151, size=256)) + [0] * 256 + list(r.integers(0, 151, size=88))
    lengths = [int(x) for x in lengths]
    inp = synth.varlen_inputs(lengths, 2, 128, 128, 64, dtype="bf16", seed=32, init_std=0.1)
    o, kf, vf = _run(gsa, torch, inp, cps)
    ro, rk, rv = _oracle_each(inp)
    errs = [rel_err(to_np(o), ro), rel_err(to_np(kf), rk), rel_err(to_np(vf), rv)]
    print("600 sequences cps=%d: o %.2e kf %.2e vf %.2e" % (cps, *errs))
    assert max(errs) <= TOL["bf16"]
    assert np.array_equal(to_np(kf)[256:512], inp["k0"].f64[256:512])


def test_varlen_at_the_unit_limit(gsa, torch):
    """257 sequences x 255 heads: a first group of 256 sequences fills 65280
    grid rows (at most 65535 are taken), the last sequence runs alone; the
    forward and the backward of the packed batch, checked on sampled
    sequences (every head); one head more is rejected on the host."""
    r = np.random.default_rng(41)
    lengths = [int(x) for x in r.integers(0, 41, size=257)]
    lengths[0], lengths[255], lengths[256] = 40, 1, 70
    H, d, m = 255, 64, 32
    inp = synth.varlen_inputs(lengths, H, d, d, m, dtype="bf16", seed=42, init_std=0.1)
    o, kf, vf = _run(gsa, torch, inp)
    cu = inp["cu_seqlens"]
    worst = 0.0
    for s_ in (0, 128, 255, 256):
        k0, v0 = inp["k0"].f64[s_:s_ + 1], inp["v0"].f64[s_:s_ + 1]
        ref = oracle.gsa_fwd(*(_seq(inp[x].f64, cu, s_) for x in "qkvg"), k0, v0, tau=8.0,
                             nthreads=oracle.max_threads())
        if lengths[s_]:
            worst = max(worst, rel_err(_seq(to_np(o), cu, s_), ref["o"]))
        worst = max(worst, rel_err(to_np(kf)[s_:s_ + 1], ref["kf"]), rel_err(to_np(vf)[s_:s_ + 1], ref["vf"]))
    print("varlen 257 sequences x H255: forward worst rel err %.2e" % worst)
    assert worst <= TOL["bf16"]
    # the backward of the same packed batch
    gi = synth.varlen_grad_inputs(lengths, H, d, d, m, dtype="bf16", seed=43)
    dev = {x: to_dev(inp[x], torch) for x in ("q", "k", "v", "g", "k0", "v0")}
    grads = gsa.gsa_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["g"], to_dev(gi["do"], torch), cu,
                               dev["k0"], dev["v0"])
    torch.cuda.synchronize()
    worst = 0.0
    for s_ in (0, 128, 255, 256):
        if not lengths[s_]:
            continue
        k0, v0 = inp["k0"].f64[s_:s_ + 1], inp["v0"].f64[s_:s_ + 1]
        ref = oracle.gsa_bwd(*(_seq(inp[x].f64, cu, s_) for x in "qkvg"), _seq(gi["do"].f64, cu, s_),
                             k0, v0, tau=8.0, nthreads=oracle.max_threads())
        for name, x in zip(("dq", "dk", "dv", "dg"), grads[:4]):
            worst = max(worst, rel_err(_seq(to_np(x), cu, s_), ref[name]))
    print("varlen 257 sequences x H255: backward worst rel err %.2e" % worst)
    assert worst <= TOL["bf16"]
    # one head more and the first group would need 65536 grid rows: rejected on
    # the host before anything is launched
    n = 257
    x = torch.zeros((H + 1, n, d), dtype=torch.bfloat16, device="cuda")
    gx = torch.zeros((H + 1, n, m), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gsa.GsaError):
        gsa.gsa_fwd_varlen(x, x, x, gx, np.arange(n + 1, dtype=np.int32))
