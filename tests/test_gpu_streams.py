"""The library keeps no mutable state between calls (each call's scratch is
its own workspace): forwards and backwards launched on several streams at
once, from one host thread or from several, give the bits of the same calls
run one after another."""
import threading

import pytest

import synth
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "k0", "v0")
# (B, H, T, d, m): several segments per unit, ragged tails, both head sizes
SHAPES = [(2, 4, 1000, 128, 64), (1, 8, 3000, 128, 64), (3, 2, 777, 64, 32), (2, 2, 1500, 128, 128)]


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


def _problems(torch):
    probs = []
    for i, (B, H, T, d, m) in enumerate(SHAPES):
        inp = synth.gsa_inputs(B, H, T, d, d, m, dtype="bf16", seed=70 + i, init_std=0.1)
        gi = synth.gsa_grad_inputs(B, H, T, d, d, m, dtype="bf16", seed=170 + i, final_std=0.1)
        dev = {n: to_dev(inp[n], torch) for n in NAMES}
        dev["do"] = to_dev(gi["do"], torch)
        dev["dkf"] = to_dev(gi["dkf"], torch)
        dev["dvf"] = to_dev(gi["dvf"], torch)
        probs.append(dev)
    return probs


def _fwd(gsa, p):
    return gsa.gsa_fwd(*(p[n] for n in NAMES), final_state=True)


def _bwd(gsa, p):
    return gsa.gsa_bwd(p["q"], p["k"], p["v"], p["g"], p["do"], p["k0"], p["v0"], p["dkf"], p["dvf"],
                       state_grads=True)


def _same(a, b, label):
    for i, (x, y) in enumerate(zip(a, b)):
        assert (x is None) == (y is None), (label, i)
        if x is not None:
            assert x.shape == y.shape and bool((x == y).all()), (label, i)


def test_concurrent_streams_match_sequential(gsa, torch):
    probs = _problems(torch)
    ref_f = [_fwd(gsa, p) for p in probs]
    ref_b = [_bwd(gsa, p) for p in probs]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(2 * len(probs))]
    got_f, got_b = [], []
    for i, p in enumerate(probs):
        for s in streams[2 * i: 2 * i + 2]:
            s.wait_stream(main)
        with torch.cuda.stream(streams[2 * i]):
            got_f.append(_fwd(gsa, p))
        with torch.cuda.stream(streams[2 * i + 1]):
            got_b.append(_bwd(gsa, p))
    torch.cuda.synchronize()
    for i in range(len(probs)):
        _same(got_f[i], ref_f[i], "fwd %d" % i)
        _same(got_b[i], ref_b[i], "bwd %d" % i)


def test_concurrent_host_threads_match_sequential(gsa, torch):
    probs = _problems(torch)
    ref = [(_fwd(gsa, p), _bwd(gsa, p)) for p in probs]
    torch.cuda.synchronize()
    got = [None] * len(probs)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                out = []
                for _ in range(3):  # the calls of one thread interleave with the others'
                    out.append((_fwd(gsa, probs[i]), _bwd(gsa, probs[i])))
            s.synchronize()
            got[i] = out
        except Exception as e:  # reported below, on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(len(probs)):
        for rep, (f, b) in enumerate(got[i]):
            _same(f, ref[i][0], "thread %d fwd %d" % (i, rep))
            _same(b, ref[i][1], "thread %d bwd %d" % (i, rep))
