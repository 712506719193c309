"""The no-allocation forward inside a captured HIP graph (what it is for):
captured once, then replayed with new inputs copied into the captured
buffers, eager work and synchronisations between the replays; every replay
must give the bits of an eager gsa_fwd on the same inputs."""
import pytest

import synth
from tests.gpu_helpers import to_dev

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


@pytest.mark.parametrize("B,H,T,m", [(2, 4, 1000, 64), (1, 2, 300, 128)])
def test_noalloc_forward_replays_in_a_graph(gsa, torch, B, H, T, m):
    names = ("q", "k", "v", "g", "k0", "v0")
    sets = [synth.gsa_inputs(B, H, T, 128, 128, m, dtype="bf16", seed=40 + i, init_std=0.1) for i in range(3)]
    static = {n: to_dev(sets[0][n], torch) for n in names}
    out = torch.empty_like(static["v"])
    kf = torch.empty((B, H, m, 128), dtype=torch.float32, device="cuda")
    vf = torch.empty_like(kf)

    def fwd():
        gsa.gsa_fwd_noalloc(*(static[n] for n in names), out=out, k_final=kf, v_final=vf)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()  # warm-up on the capture stream: one-time set-up happens outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    torch.cuda.synchronize()
    for rep in range(6):
        inp = sets[rep % 3]
        dev = {n: to_dev(inp[n], torch) for n in names}
        for n in names:
            static[n].copy_(dev[n])
        ref_o, ref_kf, ref_vf = gsa.gsa_fwd(*(dev[n] for n in names), final_state=True)  # eager
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), rep
        assert torch.equal(kf, ref_kf) and torch.equal(vf, ref_vf), rep
