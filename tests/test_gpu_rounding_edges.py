"""Codes for values whose scaled product lands exactly on, or within 2e-6 of, a
half-integer: the cases where the rounding mode and the float32 product
decide the code.  Rows are built on the CPU by brute force over fp16 values
(row absmax m in [64, 128), x <= m), then quantised by every GPU path -- the
single-launch decode kernel (T <= 16), the multi-kernel path and the weight
quantiser -- and compared with the oracle bit for bit.  Also bf16 rows whose
absmax lies below 2^-100 (down to subnormals), where 127 / absmax would
overflow float32, on every quantiser path."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _edge_rows(K=256, rows=16):
    xs = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    near, ties = [], []
    for mb in range(0x5400, 0x5800):
        m = np.float32(np.uint16(mb).view(np.float16))
        s = np.float32(127) / m
        x = xs[xs <= m]
        v = x * s
        frac = v - np.floor(v)
        n_sel = x[(np.abs(frac - np.float32(0.5)) < 2e-6) & (frac != np.float32(0.5))]
        t_sel = x[frac == np.float32(0.5)]
        if n_sel.size:
            near.append((m, np.concatenate([n_sel, t_sel])))
        elif t_sel.size:
            ties.append((m, t_sel))
    picked = near + ties[::max(1, len(ties) // 64)]
    rng = np.random.default_rng(5)
    out = np.zeros((rows, K), np.float32)
    for r in range(rows):
        m, sel = picked[r % len(picked)]
        vals = rng.choice(sel, size=K - 1)
        signs = np.where(rng.random(K - 1) < 0.5, -1.0, 1.0).astype(np.float32)
        out[r, 0] = m
        out[r, 1:] = vals * signs
        rng.shuffle(out[r])
    return out.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("T", [16, 5])
def test_tie_codes_activations(T, fused, monkeypatch):
    import bit_quantized_matmul_amd as B
    import torch
    monkeypatch.setenv("LLI8_FUSED_DECODE", fused)
    Xb = _edge_rows()[:T]
    X = O.decode_bits(Xb, "f16")
    ridx, rCA, rSCA = O.quantize_activations(X, 0.0)
    W = torch.randn((48, 256), dtype=torch.float16, device="cuda")
    CB, SCB = B.lli8_quant_weight_rowwise(W)
    out, ws = B.lli8_int8_linear(to_dev(Xb, "f16"), CB, SCB, None, 0.0, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(ws.SCA[:T].cpu().numpy(), rSCA)
    assert np.array_equal(ws.CA.cpu().numpy(), rCA)


def test_tie_codes_weights():
    import bit_quantized_matmul_amd as B
    import torch
    Wb = _edge_rows(K=512, rows=64)
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(Wb, "f16"))
    torch.cuda.synchronize()
    rCB, rSCB = O.quantize_weight(O.decode_bits(Wb, "f16"))
    assert np.array_equal(SCB.cpu().numpy(), rSCB)
    assert np.array_equal(CB.cpu().numpy(), rCB)


# ------------------------------------------------ rows of tiny magnitude ----
# bf16 rows whose absmax lies below 2^-100, where 127 / absmax can overflow
# float32 (the quantisers then scale the row and its absmax by 2^64 first):
# rows scaled by 2^-124 (absmax near 2^-122) and rows of subnormals, beside
# ordinary rows, through every quantiser path.

def _tiny_rows_bits(R, C, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((R, C))
    v[1::4] *= 2.0 ** -124
    bits = O.round_to_dtype_bits(v, "bf16")
    sub = rng.integers(1, 0x80, size=(R, C), dtype=np.uint16) | (rng.integers(0, 2, size=(R, C), dtype=np.uint16) << 15)
    bits[3::4] = sub[3::4]
    return bits


@pytest.mark.parametrize("K", [520, 1001])
def test_tiny_rows_weights(K):
    import bit_quantized_matmul_amd as B
    import torch
    Wb = _tiny_rows_bits(64, K, seed=K)
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(Wb, "bf16"))
    torch.cuda.synchronize()
    rCB, rSCB = O.quantize_weight(O.decode_bits(Wb, "bf16"))
    assert (rSCB[1::4] < 2.0 ** -100).all() and (rSCB[3::4] < 2.0 ** -126).all()
    assert np.array_equal(SCB.cpu().numpy(), rSCB)
    assert np.array_equal(CB.cpu().numpy(), rCB)


@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("T,K,tau", [(12, 512, 0.0), (12, 512, 6.0), (40, 1001, 6.0), (100, 520, 6.0), (300, 64, 2.5)])
def test_tiny_rows_activations(T, K, tau, fused, monkeypatch):
    """The fused decode (T <= 16), the one-launch split (T <= 32), the any-K
    quantiser (K % 8 != 0) and the register quantiser, with and without
    outlier columns; the output too."""
    import bit_quantized_matmul_amd as B
    import torch
    from tests.gpu_helpers import assert_out, bits_of
    monkeypatch.setenv("LLI8_FUSED_DECODE", fused)
    Xb = _tiny_rows_bits(T, K, seed=T + K)
    Xb[0, 7] = O.round_to_dtype_bits(np.array([9.5]), "bf16")[0]  # an outlier column from an ordinary row
    X = O.decode_bits(Xb, "bf16")
    Wb = _tiny_rows_bits(48, K, seed=7)
    CB, SCB = B.lli8_quant_weight_rowwise(to_dev(Wb, "bf16"))
    out, ws = B.lli8_int8_linear(to_dev(Xb, "bf16"), CB, SCB, None, tau, want_acc=True)
    torch.cuda.synchronize()
    rCB, rSCB = O.quantize_weight(O.decode_bits(Wb, "bf16"))
    r = O.linear_forward(Xb, "bf16", rCB, rSCB, None, tau)
    n = int(ws.n_idx.item())
    assert np.array_equal(ws.idx[:n].cpu().numpy(), r["idx"])
    assert (r["SCA"][1::4] < 2.0 ** -100).all()
    assert np.array_equal(ws.SCA[:T].cpu().numpy(), r["SCA"])
    assert np.array_equal(ws.CA.cpu().numpy(), r["CA"])
    assert np.array_equal(ws.acc.cpu().numpy(), r["acc"])
    assert_out(bits_of(out), r, "bf16")


@pytest.mark.parametrize("axis", ["rows", "cols"])
@pytest.mark.parametrize("n,length", [(64, 96), (24, 3000), (24, 5000)])
def test_tiny_vectors_vectorwise_absmax(axis, n, length):
    # n vectors of `length` values: rows held in registers (2, 8 or 24 chunks
    # per lane), columns 8 or 32 rows per thread in registers, or walked twice
    import bit_quantized_matmul_amd as B
    import torch
    Xb = _tiny_rows_bits(n, length, seed=3)
    if axis == "cols":
        Xb = np.ascontiguousarray(Xb.T)
    codes, scale, _ = B.lli8_quant_vectorwise(to_dev(Xb, "bf16"), "absmax", axis)
    torch.cuda.synchronize()
    rc, rs = O.absmax_quantize(O.decode_bits(Xb, "bf16"), 1 if axis == "rows" else 0)
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
