"""The Linear8bitLt-style module on the GPU against the CPU oracle: the
pages' conversion example (16-bit state dict in, quantisation on .to(0)), the
issue page's state.idx case, per-forward quantisation (has_fp16_weights=True),
bf16, and persistence of the int8 codes with their scales."""
import json
import os

import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import assert_out, bits_of, to_dev
from tests import parity_cases as PC
from workloads import random_case

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nn():
    from bit_quantized_matmul_amd import nn as lnn
    return lnn


def _module_from_case(case, has_fp16_weights, threshold):
    """A Linear8bitLt loaded from a torch.nn.Linear holding the case's weights."""
    import torch
    dt = torch.float16 if case.dtype == "f16" else torch.bfloat16
    fp = torch.nn.Linear(case.K, case.N, bias=case.bias is not None).to(dt)
    with torch.no_grad():
        fp.weight.copy_(to_dev(case.W, case.dtype, "cpu"))
        if case.bias is not None:
            fp.bias.copy_(to_dev(case.bias, case.dtype, "cpu"))
    m = _nn().Linear8bitLt(case.K, case.N, bias=case.bias is not None, has_fp16_weights=has_fp16_weights,
                           threshold=threshold, dtype=dt)
    m.load_state_dict(fp.state_dict())
    return m.to(0)


def _check(m, case, threshold, x_bits=None):
    import torch
    xb = case.X if x_bits is None else x_bits
    x = to_dev(xb, case.dtype)
    with torch.no_grad():
        out = m(x)
    torch.cuda.synchronize()
    CB, SCB = O.quantize_weight_bits(case.W, case.dtype)
    r = O.linear_forward(xb, case.dtype, CB, SCB, case.bias, threshold)
    used_CB = m.weight.CB if m.is_quantized else m.state.CB
    used_SCB = m.weight.SCB if m.is_quantized else m.state.SCB
    assert np.array_equal(used_CB.cpu().numpy(), CB), "CB"
    assert np.array_equal(used_SCB.cpu().numpy(), SCB), "SCB"
    assert np.array_equal(m.state.idx.cpu().numpy(), r["idx"]), "state.idx"
    assert np.array_equal(m.state.ws.CA.cpu().numpy(), r["CA"]), "CA"
    assert_out(bits_of(out), r, case.dtype)
    return out, r


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("has_fp16_weights", [False, True])
@pytest.mark.parametrize("threshold", PC.MODULE_THRESHOLDS)
def test_module_matches_oracle(dtype, has_fp16_weights, threshold):
    case = PC.module_case(dtype)
    m = _module_from_case(case, has_fp16_weights, threshold)
    assert m.is_quantized == (not has_fp16_weights)
    if not has_fp16_weights:
        assert m.weight.dtype.is_floating_point is False and m.weight.CB.dtype.itemsize == 1
    _, r = _check(m, case, threshold)
    if threshold == 0.0:
        assert r["idx"].size == 0


def test_conversion_example_sequential():
    """Two Linear8bitLt(64, 64) loaded from an fp16 nn.Sequential, quantised on .to(0)."""
    import torch
    torch.manual_seed(0)
    fp16_model = torch.nn.Sequential(torch.nn.Linear(64, 64), torch.nn.Linear(64, 64)).half()
    lnn = _nn()
    int8_model = torch.nn.Sequential(lnn.Linear8bitLt(64, 64, has_fp16_weights=False, threshold=6.0),
                                     lnn.Linear8bitLt(64, 64, has_fp16_weights=False, threshold=6.0))
    int8_model.load_state_dict(fp16_model.state_dict())
    int8_model = int8_model.to(0)
    for layer, ref in zip(int8_model, fp16_model):
        assert layer.weight.dtype == torch.int8 and layer.SCB.dtype == torch.float32
        CB, SCB = O.quantize_weight_bits(ref.weight.detach().view(torch.int16).numpy().view(np.uint16), "f16")
        assert np.array_equal(layer.weight.CB.cpu().numpy(), CB)
        assert np.array_equal(layer.weight.SCB.cpu().numpy(), SCB)
        rec = layer.recovered_weight().float().cpu().numpy()
        np.testing.assert_array_equal(rec, O.recover_weight(CB, SCB, "f16"))
        assert np.all(np.abs(rec - ref.weight.detach().float().numpy()) <= SCB[:, None] / 254 + 1e-3)
    x = torch.randn(8, 64, dtype=torch.float16)
    x[:, 5] *= 20
    with torch.no_grad():
        y = int8_model(x.cuda())
    torch.cuda.synchronize()
    # the oracle, layer by layer, feeding the GPU's first-layer output forward
    xb = x.view(torch.int16).numpy().view(np.uint16)
    h = int8_model[0](x.cuda())
    for layer, ref, inp in ((int8_model[0], fp16_model[0], xb), (int8_model[1], fp16_model[1], bits_of(h))):
        CB, SCB = O.quantize_weight_bits(ref.weight.detach().view(torch.int16).numpy().view(np.uint16), "f16")
        bias = ref.bias.detach().view(torch.int16).numpy().view(np.uint16)
        r = O.linear_forward(inp, "f16", CB, SCB, bias, 6.0)
        got = layer(to_dev(inp, "f16"))
        assert_out(bits_of(got), r, "f16")
    assert 5 in int8_model[0].state.idx.cpu().tolist()
    assert y.shape == (8, 64)


def test_issue_state_idx_all_columns():
    """Linear8bitLt(8, 4, has_fp16_weights=False, threshold=0.1), x [2, 8] ~ N(0, 1):
    state.idx lists every column, as the issue page reports."""
    import torch
    g = json.load(open(os.path.join(GOLDEN, "issue_all_columns_flagged.json")))
    torch.manual_seed(42)
    linear_fp = torch.nn.Linear(g["in_features"], g["out_features"]).half()
    m = _nn().Linear8bitLt(g["in_features"], g["out_features"], has_fp16_weights=False,
                           threshold=g["threshold"])
    m.load_state_dict(linear_fp.state_dict())
    m = m.to(0)
    # a seeded N(0, 1) draw in which, as in the issue's, every column has some
    # |x| > 0.1 (torch's own generator does not reproduce the reporter's draw)
    x = np.random.default_rng(1609).standard_normal(g["x_shape"]).astype(np.float16)
    assert (np.abs(x.astype(np.float32)) > g["threshold"]).any(axis=0).all()
    with torch.no_grad():
        _ = m(torch.from_numpy(x).cuda())
    assert m.state.idx.cpu().numpy().tolist() == g["state_idx_printed"]
    assert O.outlier_columns(x.astype(np.float32), g["threshold"]).tolist() == g["state_idx_printed"]


def test_fp16_weights_requantised_every_forward():
    import torch
    case = PC.module_requant_case()
    m = _module_from_case(case, True, 6.0)
    _check(m, case, 6.0)
    with torch.no_grad():
        m.weight.mul_(-2.0)  # exact in fp16
    W2 = O.round_to_dtype_bits(-2.0 * O.decode_bits(case.W, "f16").astype(np.float32), "f16")
    case.W = W2
    _check(m, case, 6.0)


def test_persistence_round_trip_is_bit_identical(tmp_path):
    import torch
    lnn = _nn()
    case = random_case(20, 96, 40, seed=17, n_out=2)
    m = _module_from_case(case, False, 6.0)
    x = to_dev(case.X, "f16")
    with torch.no_grad():
        y1 = m(x)
    p = str(tmp_path / "int8.safetensors")
    lnn.save_int8(m, p)
    m2 = lnn.Linear8bitLt(case.K, case.N, has_fp16_weights=False, threshold=6.0)
    m2.load_state_dict(lnn.load_int8(p))
    m2 = m2.cuda()
    with torch.no_grad():
        y2 = m2(x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(m2.weight.CB, m.weight.CB) and torch.equal(m2.SCB, m.SCB)


def test_leading_dims_and_workspace_reuse():
    import torch
    case = PC.module_reuse_case()
    m = _module_from_case(case, False, 6.0)
    x = to_dev(case.X, "f16").reshape(2, 3, 4, 64)
    with torch.no_grad():
        y = m(x)
        ws = m.state.ws
        y_again = m(x)
    assert y.shape == (2, 3, 4, 16) and m.state.ws is ws and torch.equal(y, y_again)
    _check(m, case, 6.0)
