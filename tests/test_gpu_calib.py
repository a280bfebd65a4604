"""The matrix-core calibration loop (not a step of the method).

Pattern 0 (every operand byte 1): every thread's accumulators sum to 4096
per iteration (32 products of ones per instruction, 8 instructions, 16
accumulators each).  Pattern 1 (pseudo-random bytes, defined in the C
header): the sums are recomputed here from that definition.  Within a wave
the A and B operands of one instruction share their layout -- lanes l and
l + 32 hold the same rows, each byte position b of a lane's 16 bytes stands
for one k -- so the sum of the whole 32 x 32 product over the wave is
sum over (lane half, byte) of (column sum of A) x (column sum of B), which
needs no knowledge of which k a byte position is.  The reported operation
count is the launch's."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _mix(x):
    x = x.astype(np.uint32)
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    return x


def _random_pattern_wave_sums(n_threads, iters):
    """Per-wave sums (mod 2^32) of the threads' accumulator sums for pattern 1."""
    t = np.arange(n_threads, dtype=np.uint32)[:, None]
    e = np.arange(4, dtype=np.uint32)[None, :]
    waves = n_threads // 64
    total = np.zeros(waves, dtype=np.int64)
    ops_a, ops_b = [], []
    for j in range(4):
        a = _mix(32 * t + 4 * j + e).view(np.int8).reshape(waves, 2, 32, 16).astype(np.int64)
        b = _mix(32 * t + 16 + 4 * j + e).view(np.int8).reshape(waves, 2, 32, 16).astype(np.int64)
        ops_a.append(a.sum(axis=2))  # [wave, lane half, byte]: column sums over the 32 rows
        ops_b.append(b.sum(axis=2))
    for c in range(8):
        total += (ops_a[c % 4] * ops_b[c // 2]).sum(axis=(1, 2))
    return (total * iters) % (1 << 32)


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


@pytest.mark.parametrize("iters", [1, 3, 1000])
def test_mfma_loop_random_operands(iters):
    import torch
    import bit_quantized_matmul_amd as B
    sink, ops = B.lli8_mfma_i8_loop(iters, pattern=1)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.int64).reshape(-1, 64).sum(axis=1) % (1 << 32)
    want = _random_pattern_wave_sums(sink.numel(), iters)
    assert np.array_equal(got, want)
    assert ops == sink.numel() // 64 * 8 * 2 * 32 ** 3 * iters
