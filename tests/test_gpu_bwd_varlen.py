"""GPU parity of the backward over a packed batch of variable-length sequences
(gsa_bwd_varlen, through the C ABI): each sequence is an independent run of
the method, so the oracle is the float64 backward on each sequence's own
slice.  Bar: max |x - y| / max |y| per gradient tensor <= 2e-2 for bfloat16
inputs, 1e-4 for float32."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import RawEvents, TOL, rel_err, to_dev, to_np

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


def _seq(x, cu, s):
    return x[:, cu[s]:cu[s + 1]][None]


def _oracle_each(inp, gi, tau=8.0):
    cu = inp["cu_seqlens"]
    n = len(cu) - 1
    H, total, dk = inp["q"].shape
    dv, m = inp["v"].shape[-1], inp["g"].shape[-1]
    out = dict(dq=np.zeros((H, total, dk)), dk=np.zeros((H, total, dk)), dv=np.zeros((H, total, dv)),
               dg=np.zeros((H, total, m)), dk0=np.zeros((n, H, m, dk)), dv0=np.zeros((n, H, m, dv)))
    opt = lambda x, s: None if x is None else x.f64[s:s + 1]
    for s in range(n):
        r = oracle.gsa_bwd(*(_seq(inp[x].f64, cu, s) for x in "qkvg"), _seq(gi["do"].f64, cu, s),
                           opt(inp["k0"], s), opt(inp["v0"], s), opt(gi["dkf"], s), opt(gi["dvf"], s),
                           tau=tau, nthreads=oracle.max_threads())
        for name in ("dq", "dk", "dv", "dg"):
            out[name][:, cu[s]:cu[s + 1]] = r[name][0]
        out["dk0"][s], out["dv0"][s] = r["dk0"][0], r["dv0"][0]
    return out


def _run(gsa, torch, inp, gi):
    dev = {x: to_dev(inp[x], torch) for x in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {x: to_dev(gi[x], torch) for x in ("do", "dkf", "dvf")}
    out = gsa.gsa_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"], inp["cu_seqlens"],
                             dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True)
    torch.cuda.synchronize()
    return dict(zip(GRADS, out))


def _check(gsa, torch, lengths, H, d, m, dtype, init, final, seed):
    inp = synth.varlen_inputs(lengths, H, d, d, m, dtype=dtype, seed=seed,
                              init_std=0.1 if init else None)
    gi = synth.varlen_grad_inputs(lengths, H, d, d, m, dtype=dtype, seed=seed + 500,
                                  final_std=1.0 if final else None)
    got = _run(gsa, torch, inp, gi)
    ref = _oracle_each(inp, gi)
    errs = {nm: rel_err(to_np(got[nm]), ref[nm]) if ref[nm].size else 0.0 for nm in GRADS}
    print("gsa_bwd_varlen n=%d H%d d%d m%d %s: %s" % (len(lengths), H, d, m, dtype,
                                                      " ".join("%s %.2e" % kv for kv in errs.items())))
    assert max(errs.values()) <= TOL[dtype], errs
    return inp, gi, got


MIX = [0, 1, 63, 64, 65, 200, 1000, 130, 0, 7]


@pytest.mark.parametrize("dtype,d,m", [("bf16", 128, 64), ("f32", 64, 32)])
def test_bwd_varlen_mixed_lengths(gsa, torch, dtype, d, m):
    """Empty, one-token, sub-chunk, exact-chunk, ragged and multi-chunk
    sequences in one call, with initial states and final-state gradients."""
    inp, gi, got = _check(gsa, torch, MIX, 2, d, m, dtype, init=True, final=True, seed=1)
    for s, L in enumerate(MIX):   # an empty sequence passes its final-state gradients through
        if L == 0:
            assert np.array_equal(to_np(got["dk0"])[s], gi["dkf"].f64[s])


def test_bwd_varlen_no_states(gsa, torch):
    _check(gsa, torch, [300, 17, 0, 129], 3, 128, 64, "bf16", init=False, final=False, seed=2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_varlen_equal_lengths_is_the_dense_call(gsa, torch, dtype):
    """Equal lengths: in float32 the packed backward gives the dense
    backward's bits (the same token-walk kernels); in bf16 the dense call runs
    the chunk form on the matrix cores and the packed one the token walks, so
    both are held to the oracle at the bf16 bar instead."""
    B, H, T = 3, 2, 300
    dense = synth.gsa_inputs(B, H, T, 128, 128, 64, dtype=dtype, seed=8, init_std=0.1)
    gi = synth.gsa_grad_inputs(B, H, T, 128, 128, 64, dtype=dtype, seed=9, final_std=1.0)
    dev = {x: to_dev(dense[x], torch) for x in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {x: to_dev(gi[x], torch) for x in ("do", "dkf", "dvf")}
    a = gsa.gsa_bwd(dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"], dev["k0"], dev["v0"],
                    ddev["dkf"], ddev["dvf"], state_grads=True)
    pk = {x: t.permute(1, 0, 2, 3).reshape(H, B * T, -1).contiguous()
          for x, t in (("q", dev["q"]), ("k", dev["k"]), ("v", dev["v"]), ("g", dev["g"]),
                       ("do", ddev["do"]))}
    b = gsa.gsa_bwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["do"], [i * T for i in range(B + 1)],
                           dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True)
    torch.cuda.synchronize()
    b = [y.reshape(H, B, T, -1).permute(1, 0, 2, 3) for y in b[:4]] + list(b[4:])
    if dtype == "f32":
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        return
    ref = oracle.gsa_bwd(*(dense[n].f64 for n in "qkvg"), gi["do"].f64, dense["k0"].f64,
                         dense["v0"].f64, gi["dkf"].f64, gi["dvf"].f64, tau=8.0,
                         nthreads=oracle.max_threads())
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dk0", "dv0"), a, b):
        ex, ey = rel_err(to_np(x), ref[name]), rel_err(to_np(y), ref[name])
        print("equal lengths %s: dense %.2e packed %.2e" % (name, ex, ey))
        assert ex <= TOL["bf16"] and ey <= TOL["bf16"], (name, ex, ey)


def test_bwd_varlen_more_than_256_sequences(gsa, torch):
    """600 sequences run as three groups; the middle group holds only empty
    sequences (their initial-state gradients are the final-state ones)."""
    r = np.random.default_rng(31)
    lengths = [int(x) for x in list(r.integers(1, 151, size=256)) + [0] * 256 +
               list(r.integers(0, 151, size=88))]
    inp, gi, got = _check(gsa, torch, lengths, 2, 128, 64, "bf16", init=True, final=True, seed=32)
    assert np.array_equal(to_np(got["dk0"])[256:512], gi["dkf"].f64[256:512])


def test_bwd_varlen_all_empty(gsa, torch):
    lengths = [0, 0, 0]
    gi = synth.varlen_grad_inputs(lengths, 2, 128, 128, 64, dtype="bf16", seed=3, final_std=1.0)
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    eg = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    dkf, dvf = to_dev(gi["dkf"], torch), to_dev(gi["dvf"], torch)
    ev = RawEvents()
    evs = ev.create(4)
    out = gsa.gsa_bwd_varlen(e, e, e, eg, e, [0, 0, 0, 0], None, None, dkf, dvf, state_grads=True,
                             events=evs)
    torch.cuda.synchronize()
    assert torch.equal(out[4], dkf) and torch.equal(out[5], dvf)
    for a, b in ((0, 1), (2, 3), (0, 3)):  # every timing hook was recorded
        assert ev.elapsed(evs[a], evs[b]) >= 0.0
