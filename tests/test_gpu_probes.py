"""GPU checks of the measurement aids (the probe kernels whose timing the benchmark
reports beside the published peaks): the copy probe copies exactly, the MFMA probe
reports the operations it enqueued, and both reject invalid arguments before launching."""

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    from quantized_linear_moe_amd import _libqe
    return _libqe


def test_probe_copy_is_exact(L):
    n = (1 << 20) + 48  # bytes, not a multiple of the grid stride
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    L.qe_probe_copy(src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_reports_its_operations(L):
    blocks, iters = 8, 3
    sink = torch.zeros(blocks * 256 * 4, dtype=torch.int32, device=DEV)
    ops = L.qe_probe_mfma_i8(sink, blocks, iters, 1)
    torch.cuda.synchronize()
    assert ops == 2 * 16 * 16 * 64 * 8 * iters * 4 * blocks
    assert int(torch.count_nonzero(sink)) > 0  # the accumulators reached the sink


def test_probe_argument_errors(L):
    buf = torch.zeros(64, dtype=torch.int32, device=DEV)
    with pytest.raises(L.QEError):
        L.qe_probe_mfma_i8(buf, 0, 1)
    with pytest.raises(L.QEError):
        L.qe_probe_mfma_i8(buf, 1, 1, 2)  # unknown operand set
    with pytest.raises(L.QEError):
        L.qe_probe_copy(buf, buf, 32)  # overlapping
    other = torch.zeros(64, dtype=torch.int32, device=DEV)
    with pytest.raises(L.QEError):
        L.qe_probe_copy(buf, other, 20)  # not a multiple of 16


def test_probe_mfma_bf16_reports_its_operations(L):
    blocks, iters = 8, 3
    sink = torch.zeros(blocks * 256 * 4, dtype=torch.float32, device=DEV)
    flops = L.qe_probe_mfma_bf16(sink, blocks, iters, 0)
    torch.cuda.synchronize()
    assert flops == 2 * 16 * 16 * 32 * 8 * iters * 4 * blocks
    # constant operands: every lane's four outputs are sums of 8 accumulators, each
    # iters times a row of A (1, 2, 3, 4 repeated) against a column of B (1, 2 repeated)
    assert torch.all(sink == sink[0]) and float(sink[0]) == 8 * iters * 8 * (1 * 1 + 2 * 2 + 3 * 1 + 4 * 2)
    with pytest.raises(L.QEError):
        L.qe_probe_mfma_bf16(sink, 1, 1, 2)
