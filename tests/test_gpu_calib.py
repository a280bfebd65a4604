"""The matrix-core calibration loop (not a step of the method): every thread's
accumulators sum to 4096 per iteration (32 products of ones per instruction,
8 instructions, 16 accumulators each), and the reported operation count is
the launch's."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [1, 3, 1000, 600000])
def test_mfma_loop_sums_and_operation_count(iters):
    import torch
    import bit_quantized_matmul_amd as B
    sink, ops = B.lli8_mfma_i8_loop(iters)
    torch.cuda.synchronize()
    expect = ((4096 * iters + 2 ** 31) % 2 ** 32) - 2 ** 31  # int32 wrap-around
    assert torch.equal(sink, torch.full_like(sink, expect))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert sink.numel() == 512 * cus
    assert ops == cus * 8 * 8 * 2 * 32 ** 3 * iters
