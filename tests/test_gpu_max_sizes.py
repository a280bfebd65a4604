"""The largest K the int32 accumulator allows (133144: K * 127^2 < 2^31), on
each kernel path that takes it: the extreme accumulator value itself, the
non-fused decode kernel (K % 16 == 0), and the large-tile 2-slot path checked
on sampled rows and columns."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import assert_out, bits_of, to_dev
from tests import parity_cases as PC

pytestmark = pytest.mark.gpu

KMAX = PC.KMAX


def _lib():
    import bit_quantized_matmul_amd as B
    return B


def test_extreme_accumulator_at_max_k():
    """Every activation and weight value +-0.25 with matching signs: every code
    is +-127 and every product +127^2, so acc = 133144 * 16129 = 2147117104;
    the output, 133144 / 16, still fits fp16."""
    import torch
    B = _lib()
    T, N = 3, 5
    rng = np.random.default_rng(7)
    signs = np.where(rng.random(KMAX) < 0.5, -0.25, 0.25).astype(np.float32)
    X = np.tile(signs, (T, 1)).astype(np.float16)
    W = np.tile(signs, (N, 1)).astype(np.float16)
    W[1] *= -1  # row 1: every product -127^2
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    CB, SCB = B.lli8_quant_weight_rowwise(Wd)
    out, ws = B.lli8_int8_linear(Xd, CB, SCB, None, 6.0, want_acc=True)
    torch.cuda.synchronize()
    acc = ws.acc.cpu().numpy()
    assert int(ws.n_idx.item()) == 0
    assert np.all(acc[:, [0, 2, 3, 4]] == KMAX * 127 * 127) and np.all(acc[:, 1] == -KMAX * 127 * 127)
    Xb = X.view(np.uint16)
    CBr, SCBr = O.quantize_weight_bits(W.view(np.uint16), "f16")
    r = O.linear_forward(Xb, "f16", CBr, SCBr, None, 6.0)
    assert np.array_equal(acc, r["acc"])
    assert_out(bits_of(out), r, "f16")


@pytest.mark.parametrize("T,K,N", PC.MAX_K_SHAPES)
def test_random_at_max_k(T, K, N):
    """K % 16 == 0 at T <= 16: the non-fused decode kernel; K % 16 != 0: the
    small-tile kernel with its ragged K tail."""
    import torch
    B = _lib()
    case = PC.max_k_case(T, K, N)
    X = to_dev(case.X, "f16")
    W = to_dev(case.W, "f16")
    bias = to_dev(case.bias, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out, ws = B.lli8_int8_linear(X, CB, SCB, bias, case.threshold, want_acc=True)
    torch.cuda.synchronize()
    CBr, SCBr = O.quantize_weight_bits(case.W, "f16")
    assert np.array_equal(CB.cpu().numpy(), CBr) and np.array_equal(SCB.cpu().numpy(), SCBr)
    r = O.linear_forward(case.X, "f16", CBr, SCBr, case.bias, case.threshold)
    n = int(ws.n_idx.item())
    assert np.array_equal(ws.idx[:n].cpu().numpy(), r["idx"])
    assert np.array_equal(ws.CA.cpu().numpy(), r["CA"])
    assert np.array_equal(ws.acc.cpu().numpy(), r["acc"])
    assert_out(bits_of(out), r, "f16")


def test_large_tiles_at_large_k_sampled():
    """T, N >= 512 and K = 133120 (a multiple of 256: the 2-slot direct-load
    ring) with ragged T and N; accumulators and outputs on sampled rows and
    columns, the activation split in full."""
    import torch
    B = _lib()
    T, K, N = 520, 133120, 600
    case = PC.large_k_tiles_case()
    X = to_dev(case.X, "f16")
    W = to_dev(case.W, "f16")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    del W
    out, ws = B.lli8_int8_linear(X, CB, SCB, None, case.threshold, want_acc=True)
    torch.cuda.synchronize()
    rows, cols = PC.LARGE_K_ROWS, PC.LARGE_K_COLS
    sCB, sSCB = O.quantize_weight_bits(case.W, "f16", rows=cols)
    assert np.array_equal(CB[torch.from_numpy(cols).cuda()].cpu().numpy(), sCB)
    CBs = np.zeros((N, K), np.int8)
    SCBs = np.zeros(N, np.float32)
    CBs[cols], SCBs[cols] = sCB, sSCB
    r = O.linear_forward(case.X, "f16", CBs, SCBs, None, case.threshold, rows=rows, cols=cols)
    n = int(ws.n_idx.item())
    assert np.array_equal(ws.idx[:n].cpu().numpy(), r["idx"])
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    assert np.array_equal(ws.CA[ri].cpu().numpy(), r["CA"])
    assert np.array_equal(ws.acc[ri][:, ci].cpu().numpy(), r["acc"])
    assert_out(bits_of(out[ri][:, ci]), r, "f16")
