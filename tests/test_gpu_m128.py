"""GPU parity at m = 128 slots against the float64 oracle (which runs the plain
recurrence over all 128 slots).  In bfloat16 the forward runs the slots as two
groups of 64, each with its own chunk form, and merges the groups' outputs by
their log-sum-exps; the tests cover the merge on every read, the exact
recurrence of a strongly decaying chunk inside one group, the segment splits
and the final states (slot rows of both groups).  Bar: max |x - y| / max |y|
per tensor <= 2e-2 (bf16 inputs), 1e-4 (float32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

M = 128


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


def _check(gsa, torch, B, H, T, d, dtype="bf16", init=True, cps=0, seed=0, mutate=None, nl="softmax",
           tau=8.0):
    inp = synth.gsa_inputs(B, H, T, d, d, M, dtype=dtype, seed=seed, init_std=0.1 if init else None)
    if mutate is not None:
        mutate(inp)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, to_dev(inp["k0"], torch), to_dev(inp["v0"], torch), tau=tau,
                            final_state=True, chunks_per_segment=cps, nonlinearity=nl)
    torch.cuda.synchronize()
    opt = lambda x: None if x is None else x.f64
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), opt(inp["k0"]), opt(inp["v0"]), tau=tau,
                         nonlinearity=nl, nthreads=oracle.max_threads())
    errs = (rel_err(to_np(o), ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"]))
    print("m128 B%d H%d T%d d%d %s %s cps=%d: o %.2e kf %.2e vf %.2e" % ((B, H, T, d, dtype, nl, cps) + errs))
    assert max(errs) <= TOL[dtype], errs


def test_supported(gsa):
    assert gsa.gsa_fwd_supported(128, 128, M, 64, gsa.DTYPE_BF16)
    assert gsa.gsa_fwd_supported(64, 64, M, 64, gsa.DTYPE_BF16)
    assert gsa.gsa_decode_supported(128, 128, M, gsa.DTYPE_BF16)
    assert gsa.gsa_decode_supported(128, 128, M, gsa.DTYPE_F32)


@pytest.mark.parametrize("T", [1, 65, 200])
@pytest.mark.parametrize("d", [128, 64])
def test_fwd_lengths(gsa, torch, T, d):
    """One token, a chunk and one token, several chunks with a ragged tail."""
    _check(gsa, torch, 2, 2, T, d, init=(T != 65), seed=T + d)


@pytest.mark.parametrize("cps", [1, 2, 3, 100])
def test_fwd_segmentations(gsa, torch, cps):
    _check(gsa, torch, 1, 3, 64 * 7 + 5, 128, cps=cps, seed=3)


@pytest.mark.parametrize("nl", ["identity", "swish", "relu", "relu2"])
def test_fwd_elementwise_reads(gsa, torch, nl):
    """An element-wise read needs no normalisation: the groups' outputs add."""
    _check(gsa, torch, 1, 2, 150, 128, nl=nl, seed=11)


def test_fwd_one_group_decays_fast(gsa, torch):
    """Gate logits -12 on every slot of the second group for chunks 1 and 3
    (64-token decay products near 2^-138: those chunks run the sub-chunk form
    in that group's units only), +-inf tokens (the exact walk) and +-30
    tokens elsewhere."""
    def mut(inp):
        x = inp["g"].f64.copy()
        x[..., 64:128, 64:] = -12.0
        x[..., 192:256, 64:] = -12.0
        x[..., 10, 3] = -np.inf
        x[..., 20, 100] = np.inf
        x[..., 30:40, 70] = 30.0
        inp["g"] = synth.stored(x, inp["g"].dtype)
    _check(gsa, torch, 1, 2, 64 * 5 + 11, 128, seed=12, mutate=mut)
    _check(gsa, torch, 1, 2, 64 * 5 + 11, 128, seed=12, mutate=mut, cps=1)


def test_fwd_skewed_groups(gsa, torch):
    """The softmax mass almost all in one group on some tokens and split on
    others: large initial key states on the first group's slots only."""
    def mut(inp):
        k0 = inp["k0"].f64.copy()
        k0[:, :, :64] *= 40.0
        inp["k0"] = synth.stored(k0, "f32")
    _check(gsa, torch, 2, 1, 130, 128, seed=13, mutate=mut)


def test_fwd_final_state_in_place(gsa, torch):
    """k_final / v_final written over k0 / v0 (the decode hand-off)."""
    inp = synth.gsa_inputs(1, 2, 300, 128, 128, M, dtype="bf16", seed=14, init_std=0.1)
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    ks, vs = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, ks, vs, final_state=True, k_final=ks, v_final=vs)
    torch.cuda.synchronize()
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), inp["k0"].f64, inp["v0"].f64,
                         nthreads=oracle.max_threads())
    assert kf.data_ptr() == ks.data_ptr() and vf.data_ptr() == vs.data_ptr()
    for x, y in ((o, ref["o"]), (ks, ref["kf"]), (vs, ref["vf"])):
        assert rel_err(to_np(x), y) <= TOL["bf16"]


def test_fwd_full_shape_sampled(gsa, torch):
    """B8 H4 T2048 d128 m128 (the training shape with 128 slots), default
    segmentation; the oracle on four of the 32 (b, h) units."""
    B, H, T = 8, 4, 2048
    inp = synth.gsa_inputs(B, H, T, 128, 128, M, dtype="bf16", seed=15, qkv_scale=1 / np.sqrt(128))
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, final_state=True)
    torch.cuda.synchronize()
    idx = np.array([0, 9, 22, B * H - 1])
    sel = lambda a: a.reshape(-1, *a.shape[2:])[idx][:, None]
    ref = oracle.gsa_fwd(*(sel(inp[n].f64) for n in "qkvg"), tau=8.0, nthreads=oracle.max_threads())
    errs = (rel_err(sel(to_np(o)), ref["o"]), rel_err(sel(to_np(kf)), ref["kf"]),
            rel_err(sel(to_np(vf)), ref["vf"]))
    print("m128 full shape sampled: o %.2e kf %.2e vf %.2e" % errs)
    assert max(errs) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_decode_step(gsa, torch, dtype, d):
    inp = synth.decode_inputs(3, 5, d, d, M, dtype=dtype, seed=16)
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs)
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(*(inp[n].f64 for n in "qkvg"), inp["kstate"].f64,
                                        inp["vstate"].f64)
    assert rel_err(to_np(o), ro) <= TOL[dtype]
    assert rel_err(to_np(ks), rk) <= 1e-5 and rel_err(to_np(vs), rv) <= 1e-5


def test_prefill_then_decode(gsa, torch):
    """The forward's final states (both groups' slot rows) continue through
    decode steps exactly as the forward over the longer sequence."""
    T0, T1 = 130, 4
    inp = synth.gsa_inputs(2, 2, T0 + T1, 128, 128, M, dtype="bf16", seed=17, init_std=0.1)
    dev = {n: to_dev(inp[n], torch) for n in "qkvg"}
    ks, vs = to_dev(inp["k0"], torch), to_dev(inp["v0"], torch)
    gsa.gsa_fwd(*(dev[n][:, :, :T0].contiguous() for n in "qkvg"), ks, vs, final_state=True,
                k_final=ks, v_final=vs)
    outs = [gsa.gsa_decode_step(*(dev[n][:, :, t].contiguous() for n in "qkvg"), ks, vs)
            for t in range(T0, T0 + T1)]
    torch.cuda.synchronize()
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), inp["k0"].f64, inp["v0"].f64,
                         nthreads=oracle.max_threads())
    got = np.stack([to_np(x) for x in outs], axis=2)
    assert rel_err(got, ref["o"][:, :, T0:]) <= TOL["bf16"]
    assert rel_err(to_np(ks), ref["kf"]) <= TOL["bf16"] and rel_err(to_np(vs), ref["vf"]) <= TOL["bf16"]


# ------------------------------------------------------------- backward
GRADS = ("dq", "dk", "dv", "dg", "dk0", "dv0")


def _bwd_check(gsa, torch, B, H, T, d, init=True, final=True, seed=0, mutate=None, nl="softmax", units=None,
               qkv_scale=None):
    inp = synth.gsa_inputs(B, H, T, d, d, M, dtype="bf16", seed=seed, qkv_scale=qkv_scale,
                           init_std=0.1 if init else None)
    if mutate is not None:
        mutate(inp)
    gi = synth.gsa_grad_inputs(B, H, T, d, d, M, dtype="bf16", seed=seed + 1000,
                               final_std=1.0 if final else None)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {n: to_dev(gi[n], torch) for n in ("do", "dkf", "dvf")}
    out = gsa.gsa_bwd(dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"], dev["k0"], dev["v0"], ddev["dkf"],
                      ddev["dvf"], state_grads=True, nonlinearity=nl)
    torch.cuda.synchronize()
    got = dict(zip(GRADS, out))

    def sel(x):
        if x is None:
            return None
        return x.f64 if units is None else x.f64.reshape(-1, *x.shape[2:])[units][:, None]
    ref = oracle.gsa_bwd(*(sel(inp[n]) for n in "qkvg"), sel(gi["do"]), sel(inp["k0"]), sel(inp["v0"]),
                         sel(gi["dkf"]), sel(gi["dvf"]), tau=8.0, nthreads=oracle.max_threads(), nonlinearity=nl)
    errs = {}
    for n in GRADS:
        x = to_np(got[n])
        if units is not None:
            x = x.reshape(-1, *x.shape[2:])[units][:, None]
        errs[n] = rel_err(x, ref[n])
    print("m128 bwd B%d H%d T%d d%d %s: %s" % (B, H, T, d, nl, " ".join("%s %.2e" % kv for kv in errs.items())))
    assert max(errs.values()) <= TOL["bf16"], errs


@pytest.mark.parametrize("T", [1, 65, 200])
@pytest.mark.parametrize("d", [128, 64])
def test_bwd_lengths(gsa, torch, T, d):
    _bwd_check(gsa, torch, 2, 2, T, d, init=(T != 65), final=(T != 1), seed=T + d)


@pytest.mark.parametrize("nl", ["identity", "swish", "relu2"])
def test_bwd_elementwise_reads(gsa, torch, nl):
    """Element-wise reads: each group's gradients are its own (no log-sum-exp)."""
    _bwd_check(gsa, torch, 1, 2, 150, 128, nl=nl, seed=21)


def test_bwd_relu_read_rejected(gsa, torch):
    inp = synth.gsa_inputs(1, 1, 64, 128, 128, M, dtype="bf16", seed=22)
    gi = synth.gsa_grad_inputs(1, 1, 64, 128, 128, M, dtype="bf16", seed=23)
    dev = {n: to_dev(inp[n], torch) for n in "qkvg"}
    with pytest.raises(RuntimeError):
        gsa.gsa_bwd(dev["q"], dev["k"], dev["v"], dev["g"], to_dev(gi["do"], torch), nonlinearity="relu")


def test_bwd_one_group_decays_fast(gsa, torch):
    """Sub-chunk-form chunks in the second group only (g = -12 on its slots:
    64-token products ~2^-138), and +-inf gates (exact walks)."""
    def mut(inp):
        x = inp["g"].f64.copy()
        x[..., 64:128, 64:] = -12.0
        x[..., 10, 3] = -np.inf
        x[..., 20, 100] = np.inf
        inp["g"] = synth.stored(x, "bf16")
    _bwd_check(gsa, torch, 1, 2, 64 * 3 + 11, 128, seed=24, mutate=mut)


def test_bwd_skewed_groups(gsa, torch):
    def mut(inp):
        k0 = inp["k0"].f64.copy()
        k0[:, :, :64] *= 40.0
        inp["k0"] = synth.stored(k0, "f32")
    _bwd_check(gsa, torch, 2, 1, 130, 128, seed=25, mutate=mut)


def test_bwd_full_shape_sampled(gsa, torch):
    """B8 H4 T2048 d128 m128 in the default launch configuration; three of
    the 32 units against the oracle."""
    _bwd_check(gsa, torch, 8, 4, 2048, 128, init=False, final=False, seed=26, units=[0, 13, 31],
               qkv_scale=1 / np.sqrt(128))
