"""Seeded random cases over the compiled bf16 set, against the float64 oracle
(bar 2e-2 per tensor): the forward (every read, any split, optional states,
gate shifts, a random set of fast-forgetting slots that sends chunks to the
sub-chunk form), the backward and the training pair.  Each case prints its
parameters before it runs."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

READS = ["softmax", "softmax", "softmax", "identity", "swish", "relu", "relu2"]


def _draw(seed, bwd):
    r = np.random.default_rng(1000 + seed)
    m = int(r.choice([32, 64, 128]))
    d = int(r.choice([64, 128]))
    nl = str(r.choice([x for x in READS if not (bwd and x == "relu")]))
    if m == 128 and bwd and nl == "relu":
        nl = "softmax"
    c = dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), T=int(r.integers(1, 700)), d=d, m=m, nl=nl,
             cps=int(r.choice([0, 0, 1, 2, 3, 5])), init=bool(r.integers(0, 2)), final=bool(r.integers(0, 2)),
             shift=float(r.choice([0.0, 0.0, 2.0, -3.0])))
    # drawn last, so that the draws above are those of the earlier cases:
    # n slots (a random subset) at logits N(mean, 1); at tau = 8, mean -10
    # puts 64-token decays near 2^-115 (sub-chunk form), -25 near 2^-280 with
    # 16-token ones near 2^-70
    if r.integers(0, 2):
        c["fast"] = (int(r.choice([4, 8, 16])), float(r.choice([-10.0, -14.0, -20.0, -25.0])))
    return c


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


def _inputs(c, seed):
    inp = synth.gsa_inputs(c["B"], c["H"], c["T"], c["d"], c["d"], c["m"], dtype="bf16", seed=seed,
                           g_shift=c["shift"], init_std=0.1 if c["init"] else None)
    if "fast" in c:
        n, mean = c["fast"]
        r = np.random.default_rng(2000 + seed)
        idx = r.choice(c["m"], size=n, replace=False)
        x = inp["g"].f64.copy()
        x[..., idx] = mean + r.standard_normal(x[..., idx].shape)
        inp["g"] = synth.stored(x, "bf16")
    return inp


@pytest.mark.parametrize("seed", range(16))
def test_random_forward(gsa, torch, seed):
    c = _draw(seed, bwd=False)
    print("random forward case", seed, c, flush=True)
    inp = _inputs(c, seed)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    o, kf, vf = gsa.gsa_fwd(*(dev[n] for n in ("q", "k", "v", "g", "k0", "v0")), final_state=True,
                            chunks_per_segment=c["cps"], nonlinearity=c["nl"])
    torch.cuda.synchronize()
    opt = lambda x: None if x is None else x.f64
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), opt(inp["k0"]), opt(inp["v0"]), nonlinearity=c["nl"],
                         nthreads=oracle.max_threads())
    errs = [rel_err(to_np(o), ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"])]
    print("  rel err o/kf/vf", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL["bf16"]


@pytest.mark.parametrize("seed", range(20))
def test_random_backward_and_pair(gsa, torch, seed):
    c = _draw(seed, bwd=True)
    print("random backward case", seed, c, flush=True)
    inp = _inputs(c, seed)
    gi = synth.gsa_grad_inputs(c["B"], c["H"], c["T"], c["d"], c["d"], c["m"], dtype="bf16", seed=seed + 500,
                               final_std=1.0 if c["final"] else None)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    ddev = {n: to_dev(gi[n], torch) for n in ("do", "dkf", "dvf")}
    args = (dev["q"], dev["k"], dev["v"], dev["g"], ddev["do"])
    got = gsa.gsa_bwd(*args, dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True, nonlinearity=c["nl"])
    torch.cuda.synchronize()
    opt = lambda x: None if x is None else x.f64
    ref = oracle.gsa_bwd(*(inp[n].f64 for n in "qkvg"), gi["do"].f64, opt(inp["k0"]), opt(inp["v0"]),
                         opt(gi["dkf"]), opt(gi["dvf"]), nonlinearity=c["nl"], nthreads=oracle.max_threads())
    errs = {n: rel_err(to_np(x), ref[n]) for n, x in zip(("dq", "dk", "dv", "dg", "dk0", "dv0"), got)}
    print("  rel err", " ".join("%s %.2e" % kv for kv in errs.items()))
    assert max(errs.values()) <= TOL["bf16"], errs
    if gsa.gsa_train_supported(dev["q"], dev["v"], dev["g"], c["nl"]):
        _, _, _, st = gsa.gsa_fwd_train(*(dev[n] for n in ("q", "k", "v", "g", "k0", "v0")), nonlinearity=c["nl"])
        pair = gsa.gsa_bwd_train(*args, st, dev["k0"], dev["v0"], ddev["dkf"], ddev["dvf"], state_grads=True,
                                 nonlinearity=c["nl"])
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv", "dg", "dk0", "dv0"), pair, got):
            assert torch.equal(x, y), name
