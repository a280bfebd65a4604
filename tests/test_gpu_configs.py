"""Parity on the full-size workloads, in the launch configuration the benchmark
times.  CA, SCA, idx and the bitmap are compared in full; CB/SCB on sampled
weight rows; the int32 accumulators and the output on a sampled block of rows
and columns that the oracle computes one by one."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import assert_out, bits_of, to_dev
from tests import parity_cases as PC
from workloads import config_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", PC.FULL_CONFIGS)
def test_config_parity(name):
    import torch
    import bit_quantized_matmul_amd as B
    print(f"[config parity] {name}", flush=True)
    case = config_case(name)
    X = to_dev(case.X, case.dtype)
    W = to_dev(case.W, case.dtype)
    bias = to_dev(case.bias, case.dtype) if case.bias is not None else None
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out, ws = B.lli8_int8_linear(X, CB, SCB, bias, case.threshold, want_acc=True)
    # the benchmark's launch (no accumulator output) must give the same output bits
    out_b, ws_b = B.lli8_int8_linear(X, CB, SCB, bias, case.threshold)
    torch.cuda.synchronize()
    assert torch.equal(out, out_b)

    # weight codes on sampled rows
    wrows = PC.sample_indices(case.N, 64, 192, 1)
    rCB, rSCB = O.quantize_weight_bits(case.W, case.dtype, rows=wrows)
    assert np.array_equal(CB[torch.from_numpy(wrows).cuda()].cpu().numpy(), rCB)
    assert np.array_equal(SCB[torch.from_numpy(wrows).cuda()].cpu().numpy(), rSCB)

    # activation split, in full
    Xf = O.decode_bits(case.X, case.dtype)
    ridx, rCA, rSCA = O.quantize_activations(Xf, case.threshold)
    n = int(ws.n_idx.item())
    assert n == ridx.size
    assert np.array_equal(ws.idx[:n].cpu().numpy(), ridx)
    assert np.array_equal(ws.bitmap.cpu().numpy().view(np.uint32), O.outlier_bitmap(ridx, case.K))
    assert np.array_equal(ws.SCA[:case.T].cpu().numpy(), rSCA)
    assert np.array_equal(ws.CA.cpu().numpy(), rCA)
    del Xf, rCA

    # accumulators and outputs on a sampled block
    rows, cols = PC.config_sample(case)
    sCB, sSCB = O.quantize_weight_bits(case.W, case.dtype, rows=cols)
    CBfull_cols = np.zeros((case.N, case.K), np.int8)  # only the sampled rows are read
    SCBfull = np.zeros(case.N, np.float32)
    CBfull_cols[cols] = sCB
    SCBfull[cols] = sSCB
    r = O.linear_forward(case.X, case.dtype, CBfull_cols, SCBfull, case.bias, case.threshold,
                         rows=rows, cols=cols)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    acc = ws.acc[ri][:, ci].cpu().numpy()
    assert np.array_equal(acc, r["acc"])
    ob = bits_of(out[ri][:, ci])
    err, ratio = assert_out(ob, r, case.dtype)
    print(f"[config parity] {name}: n_idx={n} out normwise rel err={err:.3e}, "
          f"worst element {ratio:.3f} x bound", flush=True)
