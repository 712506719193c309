"""The calibration kernels the benchmark uses to measure this GPU's achievable
HBM bandwidth and bf16 MFMA rate: the copy moves the bytes exactly, and the
MFMA loop's accumulators end at their closed-form value (so the loop really
ran every iteration)."""
import pytest

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


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_hbm_copy_moves_every_byte(gsa, torch, nbytes):
    gen = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=gen, device="cuda", dtype=torch.int32)
    dst = torch.zeros_like(src)
    moved = gsa.measure_hbm(dst, src)
    torch.cuda.synchronize()
    assert moved == 2 * nbytes
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_hbm_update_in_place(gsa, torch, nbytes):
    x = torch.arange(nbytes // 4, device="cuda", dtype=torch.float32).remainder_(1000.0)
    y = x.clone()
    gsa.measure_hbm(y)
    gsa.measure_hbm(y)
    torch.cuda.synchronize()
    assert torch.equal(y, x + 2.0)


@pytest.mark.parametrize("iters", [1, 1000, 16000])
def test_mfma_loop_closed_form(gsa, torch, iters):
    sink, flops = gsa.measure_mfma_bf16(iters)
    torch.cuda.synchronize()
    assert flops == gsa.MEASURE_MFMA_WORKGROUPS * 4 * iters * 8 * 2 * 16 * 16 * 32
    expect = torch.full_like(sink, 1024.0 * iters + 496.0)
    assert torch.equal(sink, expect), (sink[:4], expect[0])
