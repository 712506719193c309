"""gsa_fwd_noalloc (the forward for callers that cannot allocate: its scratch
is the library's fixed per-GPU array) against gsa_fwd with a workspace, on
two calls in a row -- the second with a smaller problem, so the scratch still
holds the first call's larger contents -- and against the oracle.  Same
kernels and segment split as gsa_fwd, so the bits must be identical."""
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


def _case(gsa, torch, B, H, T, m, init, seed):
    print("noalloc case B%d H%d T%d m%d init=%s" % (B, H, T, m, init), flush=True)
    inp = synth.gsa_inputs(B, H, T, 128, 128, m, dtype="bf16", seed=seed,
                           init_std=0.1 if init else None)
    dev = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "k0", "v0")}
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["k0"], dev["v0"])
    ref_o, ref_kf, ref_vf = gsa.gsa_fwd(*args, final_state=True)
    out = torch.empty_like(dev["v"])
    kf = torch.empty((B, H, m, 128), dtype=torch.float32, device="cuda")
    vf = torch.empty_like(kf)
    gsa.gsa_fwd_noalloc(*args, out=out, k_final=kf, v_final=vf)
    torch.cuda.synchronize()
    assert gsa.gsa_fwd_workspace_bytes(B, H, T, 128, 128, m) > 0  # the scratch is really used
    assert torch.equal(out, ref_o)
    assert torch.equal(kf, ref_kf) and torch.equal(vf, ref_vf)
    return inp, out


def test_noalloc_matches_gsa_fwd_twice(gsa, torch):
    # first the training shape (17 MB of scratch), then a smaller ragged problem
    inp, out = _case(gsa, torch, 8, 4, 2048, 64, False, 0)
    one = {n: inp[n].f64[:1, :1] for n in "qkvg"}
    ref = oracle.gsa_fwd(one["q"], one["k"], one["v"], one["g"], tau=8.0, want_states=False)
    assert rel_err(to_np(out[:1, :1]), ref["o"]) <= TOL["bf16"]
    inp2, out2 = _case(gsa, torch, 2, 3, 700, 32, True, 1)
    ref2 = oracle.gsa_fwd(*(inp2[n].f64 for n in ("q", "k", "v", "g", "k0", "v0")), tau=8.0)
    assert rel_err(to_np(out2), ref2["o"]) <= TOL["bf16"]


def test_noalloc_rejects_oversized(gsa, torch):
    cap = gsa.lib.gsa_fwd_noalloc_scratch_bytes()
    B, H, T = 16, 4, 16384
    assert gsa.gsa_fwd_workspace_bytes(B, H, T, 128, 128, 64, chunks_per_segment=1) > cap
    q = torch.empty((B, H, T, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gsa.GsaError) as e:
        gsa.gsa_fwd_noalloc(q, q, q, g, out=torch.empty_like(q), chunks_per_segment=1)
    assert e.value.status == 8
