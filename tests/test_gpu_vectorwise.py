"""lli8_quant_vectorwise (absmax / zero-point, per row / per column) against the
oracle: codes, scales and zero points bit-exact."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import to_dev
from workloads import matrix_bits

pytestmark = pytest.mark.gpu

# Routes: rows held in registers (C <= 1024, 4096, 12288) or walked twice
# (C > 12288); a column strip's rows held in registers (8, 16 or 32 per
# thread: R <= 1024, 2048, 4096 with 32-column strips, half that with the
# 64-column strips of C >= 16384) or walked twice; C % 8 != 0 per value.
SHAPES = [(37, 136), (64, 200), (33, 13), (1, 8), (5, 1), (513, 1000), (130, 64), (7, 4096), (300, 71),
          (9, 16392), (5, 16390),  # 64-column strips (C >= 16384)
          (40, 12000), (2000, 96), (4096, 40), (4100, 24), (700, 16384), (1100, 16384)]


def _ref(bits, dtype, scheme, axis):
    X = O.decode_bits(bits, dtype)
    ax = 1 if axis == "rows" else 0
    if scheme == "absmax":
        c, a = O.absmax_quantize(X, ax)
        return c, a, None
    return O.zeropoint_quantize(X, ax)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scheme", ["absmax", "zeropoint"])
@pytest.mark.parametrize("axis", ["rows", "cols"])
@pytest.mark.parametrize("R,C", SHAPES)
def test_vectorwise_matches_oracle(R, C, axis, scheme, dtype):
    import torch
    import bit_quantized_matmul_amd as B
    bits = matrix_bits(R, C, dtype, seed=R * 31 + C)
    codes, scale, zp = B.lli8_quant_vectorwise(to_dev(bits, dtype), scheme, axis)
    torch.cuda.synchronize()
    rc, rs, rz = _ref(bits, dtype, scheme, axis)
    assert np.array_equal(codes.cpu().numpy(), rc), "codes"
    assert np.array_equal(scale.cpu().numpy(), rs), "scale"
    if scheme == "zeropoint":
        assert np.array_equal(zp.cpu().numpy(), rz), "zero point"


@pytest.mark.parametrize("axis", ["rows", "cols"])
def test_vectorwise_empty_sides(axis):
    import torch
    import bit_quantized_matmul_amd as B
    for R, C in ((0, 16), (16, 0)):
        X = torch.zeros((R, C), dtype=torch.float16, device="cuda")
        codes, scale, zp = B.lli8_quant_vectorwise(X, "zeropoint", axis)
        torch.cuda.synchronize()
        n = R if axis == "rows" else C
        assert codes.shape == (R, C) and scale.shape == (n,)
        assert not scale.cpu().numpy().any() and not zp.cpu().numpy().any()
