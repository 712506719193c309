"""The C ABI from plain C: tests/c_abi/gsa_c_client (no Python, no PyTorch in
its process) allocates device memory with the HIP runtime, runs gsa_fwd, the
backward gsa_bwd of the same call and a gsa_decode_step on the final states
in float32, then the same inputs in bfloat16 through the training pair
(gsa_fwd_train, gsa_bwd_train) and gsa_fwd_noalloc, and writes the results;
they are checked here against the float64 oracle on the same inputs (chosen
exactly representable in bfloat16): bar 1e-4 for float32 storage, 2e-2 for
bfloat16."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import rel_err

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_abi", "gsa_c_client")


def test_c_client_forward_and_decode(tmp_path):
    if not os.path.exists(CLIENT):
        pytest.fail("the C client is not built (run __graft_entry__.build())")
    B, H, T, d, m = 2, 3, 200, 64, 32
    # bf16-representable values, written as float32: both storage types see them exactly
    inp = synth.gsa_inputs(B, H, T, d, d, m, dtype="bf16", seed=11)
    tok = synth.decode_inputs(B, H, d, d, m, dtype="f32", seed=12)
    do = synth.gsa_grad_inputs(B, H, T, d, d, m, dtype="bf16", seed=13)["do"]
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(np.array([B, H, T, d, d, m], dtype=np.int32).tobytes())
        for x in (inp["q"], inp["k"], inp["v"], inp["g"], tok["q"], tok["k"], tok["v"], tok["g"], do):
            f.write(np.ascontiguousarray(x.f64, dtype=np.float32).tobytes())
    dst = tmp_path / "out.bin"
    print("running the C client: B%d H%d T%d d%d m%d" % (B, H, T, d, m), flush=True)
    r = subprocess.run([CLIENT, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    out = np.fromfile(dst, dtype=np.float32).astype(np.float64)
    U = B * H
    sizes = [U * T * d, U * m * d, U * m * d, U * d, U * m * d, U * m * d,
             U * T * d, U * T * d, U * T * d, U * T * m,
             U * T * d, U * m * d, U * m * d, U * T * d, U * T * d, U * T * d, U * T * m, U * T * d]
    assert out.size == sum(sizes)
    parts = np.split(out, np.cumsum(sizes)[:-1])
    o, kf, vf, o1, kf1, vf1, gq, gk, gv, gg = parts[:10]
    bo, bkf, bvf, bgq, bgk, bgv, bgg, bo2 = parts[10:]
    ref = oracle.gsa_fwd(*(inp[n].f64 for n in "qkvg"), tau=8.0)
    assert rel_err(o.reshape(B, H, T, d), ref["o"]) <= 1e-4
    assert rel_err(kf.reshape(B, H, m, d), ref["kf"]) <= 1e-4
    assert rel_err(vf.reshape(B, H, m, d), ref["vf"]) <= 1e-4
    ro, rk, rv = oracle.gsa_decode_step(*(tok[n].f64 for n in "qkvg"), ref["kf"], ref["vf"])
    assert rel_err(o1.reshape(B, H, d), ro) <= 1e-4
    assert rel_err(kf1.reshape(B, H, m, d), rk) <= 1e-4 and rel_err(vf1.reshape(B, H, m, d), rv) <= 1e-4
    gref = oracle.gsa_bwd(*(inp[n].f64 for n in "qkvg"), do.f64, tau=8.0)
    for name, x, shape in (("dq", gq, (B, H, T, d)), ("dk", gk, (B, H, T, d)),
                           ("dv", gv, (B, H, T, d)), ("dg", gg, (B, H, T, m))):
        err = rel_err(x.reshape(shape), gref[name])
        print("C client gsa_bwd %s rel err %.2e" % (name, err))
        assert err <= 1e-4, name
    # bf16 storage: the training pair and the no-allocation forward
    for name, x, y, shape in (("o", bo, ref["o"], (B, H, T, d)), ("kf", bkf, ref["kf"], (B, H, m, d)),
                              ("vf", bvf, ref["vf"], (B, H, m, d)), ("noalloc o", bo2, ref["o"], (B, H, T, d)),
                              ("dq", bgq, gref["dq"], (B, H, T, d)), ("dk", bgk, gref["dk"], (B, H, T, d)),
                              ("dv", bgv, gref["dv"], (B, H, T, d)), ("dg", bgg, gref["dg"], (B, H, T, m))):
        err = rel_err(x.reshape(shape), y)
        print("C client bf16 %s rel err %.2e" % (name, err))
        assert err <= 2e-2, name
