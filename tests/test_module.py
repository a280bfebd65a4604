"""The Linear8bitLt-style module without a GPU: construction, state-dict
forms (16-bit and int8 + SCB), persistence through safetensors, and that a
forward on the CPU raises instead of computing anything there."""
import numpy as np
import pytest
import torch

from bit_quantized_matmul_amd.nn import Linear8bitLt, load_int8, save_int8


def _int8_state(N, K, seed=0):
    rng = np.random.default_rng(seed)
    CB = torch.from_numpy(rng.integers(-127, 128, size=(N, K), dtype=np.int8))
    SCB = torch.from_numpy(rng.uniform(0.5, 3.0, size=N).astype(np.float32))
    bias = torch.from_numpy(rng.standard_normal(N).astype(np.float16))
    return {"weight": CB, "SCB": SCB, "bias": bias}


def test_signature_and_16bit_state_dict():
    m = Linear8bitLt(64, 32, bias=True, has_fp16_weights=False, threshold=6.0)
    assert m.weight.shape == (32, 64) and m.weight.dtype == torch.float16
    assert m.bias.shape == (32,) and not m.is_quantized and m.SCB is None
    assert set(m.state_dict()) == {"weight", "bias"}
    fp = torch.nn.Linear(64, 32).half()
    m.load_state_dict(fp.state_dict())
    assert torch.equal(m.weight.data, fp.weight.data) and torch.equal(m.bias.data, fp.bias.data)
    assert m.state.idx is None


def test_no_bias_and_index_argument():
    m = Linear8bitLt(8, 4, bias=False, index=[1, 2])
    assert m.bias is None and m.index == [1, 2]
    assert set(m.state_dict()) == {"weight"}


def test_int8_state_dict_loads_and_round_trips():
    sd = _int8_state(16, 40)
    m = Linear8bitLt(40, 16, has_fp16_weights=False)
    m.load_state_dict(sd)
    assert m.is_quantized and m.weight.dtype == torch.int8
    assert m.weight.CB is m.weight.data or torch.equal(m.weight.CB, m.weight.data)
    assert torch.equal(m.weight.data, sd["weight"]) and torch.equal(m.SCB, sd["SCB"])
    out = m.state_dict()
    assert set(out) == {"weight", "bias", "SCB"}
    assert out["SCB"].dtype == torch.float32 and torch.equal(out["SCB"], sd["SCB"])
    # casting the module leaves the codes and the fp32 scales alone
    m.half()
    assert m.weight.dtype == torch.int8 and m.SCB.dtype == torch.float32


def test_int8_state_dict_needs_scb():
    sd = _int8_state(8, 8)
    del sd["SCB"]
    m = Linear8bitLt(8, 8, has_fp16_weights=False)
    with pytest.raises(RuntimeError, match="SCB"):
        m.load_state_dict(sd)


def test_int8_state_dict_shape_mismatch():
    sd = _int8_state(8, 8)
    m = Linear8bitLt(16, 8, has_fp16_weights=False)
    with pytest.raises(RuntimeError, match="do not fit"):
        m.load_state_dict(sd)


def test_safetensors_round_trip(tmp_path):
    sd = _int8_state(12, 24, seed=3)
    m = Linear8bitLt(24, 12, has_fp16_weights=False)
    m.load_state_dict(sd)
    p = str(tmp_path / "layer.safetensors")
    save_int8(m, p)
    back = load_int8(p)
    assert set(back) == {"weight", "bias", "SCB"}
    m2 = Linear8bitLt(24, 12, has_fp16_weights=False)
    m2.load_state_dict(back)
    assert torch.equal(m2.weight.data, m.weight.data) and torch.equal(m2.SCB, m.SCB)
    assert torch.equal(m2.bias.data, m.bias.data)


def test_forward_on_cpu_raises():
    m = Linear8bitLt(8, 4)
    with pytest.raises(RuntimeError, match="GPU"):
        m(torch.zeros(2, 8, dtype=torch.float16))


def test_recovered_weight_needs_quantised_module():
    m = Linear8bitLt(8, 4)
    with pytest.raises(RuntimeError, match="not quantised"):
        m.recovered_weight()
