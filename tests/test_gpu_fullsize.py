"""Parity at the full workload sizes, in the launch configuration the
benchmark times (default segmentation).  Where the oracle would take too long
it runs on a sample of independent (batch, head) units."""
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


def _units(x, idx):
    if x is None:
        return None
    a = x.f64
    return a.reshape(-1, *a.shape[2:])[idx][:, None]


@pytest.mark.parametrize("name", ["gsa_bf16_train_T2048", "gsa_bf16_long_T16384",
                                  "gsa_bf16_train_T2048_fast_forget", "gsa_bf16_train_T2048_rapid_forget",
                                  "gsa_bf16_train_T2048_extreme_forget"])
def test_gsa_full_workload(gsa, torch, name):
    w = synth.WORKLOADS[name]
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"], fast_slots=w.get("fast_slots", 0),
                           fast_shift=w.get("fast_shift", 0.0))
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o, kf, vf = gsa.gsa_fwd(q, k, v, g, to_dev(inp["k0"], torch), to_dev(inp["v0"], torch),
                            tau=w["tau"], final_state=True)
    torch.cuda.synchronize()
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"),
                         None if inp["k0"] is None else inp["k0"].f64,
                         None if inp["v0"] is None else inp["v0"].f64,
                         tau=w["tau"], nthreads=oracle.max_threads())
    errs = [rel_err(to_np(o), ref["o"]), rel_err(to_np(kf), ref["kf"]), rel_err(to_np(vf), ref["vf"])]
    print(name, "rel err o/kf/vf:", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL[w["dtype"]]


def test_gla_full_workload_sampled_units(gsa, torch):
    w = synth.WORKLOADS["gla_bf16_T4096"]
    inp = synth.gla_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], dtype=w["dtype"], seed=0,
                           qkv_scale=w["qkv_scale"])
    q, k, v, g = (to_dev(inp[n], torch) for n in "qkvg")
    o, sf = gsa.gla_fwd(q, k, v, g, tau=w["tau"], final_state=True)
    torch.cuda.synchronize()
    idx = np.array([0, 37, 90, w["B"] * w["H"] - 1])
    ref = oracle.gla_fwd(*(_units(inp[n], idx) for n in "qkvg"), tau=w["tau"],
                         nthreads=oracle.max_threads())
    on = to_np(o).reshape(-1, w["T"], w["dv"])[idx][:, None]
    sn = to_np(sf).reshape(-1, w["dk"], w["dv"])[idx][:, None]
    e1, e2 = rel_err(on, ref["o"]), rel_err(sn, ref["sf"])
    print("gla full sampled units rel err o %.2e sf %.2e" % (e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_decode_full_workload(gsa, torch):
    w = synth.WORKLOADS["gsa_decode_N256"]
    inp = synth.decode_inputs(w["N"], w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"], seed=0,
                              qkv_scale=w["qkv_scale"], state_std=w["state_std"])
    ks, vs = to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)
    o = gsa.gsa_decode_step(*(to_dev(inp[n], torch) for n in "qkvg"), ks, vs, tau=w["tau"])
    torch.cuda.synchronize()
    ro, rk, rv = oracle.gsa_decode_step(*(inp[n].f64 for n in "qkvg"), inp["kstate"].f64,
                                        inp["vstate"].f64, tau=w["tau"],
                                        nthreads=oracle.max_threads())
    errs = [rel_err(to_np(o), ro), rel_err(to_np(ks), rk), rel_err(to_np(vs), rv)]
    print("decode full rel err o/k/v:", ["%.2e" % e for e in errs])
    assert errs[0] <= TOL["bf16"] and errs[1] <= 1e-5 and errs[2] <= 1e-5
