"""Codes for values whose scaled product lands exactly on, or within 2e-6 of, a
half-integer: the cases where the rounding mode and the float32 product
decide the code.  Rows are built on the CPU by brute force over fp16 values
(row absmax m in [64, 128), x <= m), then quantised by every GPU path -- the
single-launch decode kernel (T <= 16), the multi-kernel path and the weight
quantiser -- and compared with the oracle bit for bit."""
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
