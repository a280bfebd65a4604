"""Helpers for the parity tests: move seeded numpy inputs to the device and
compare the HIP path's results with the oracle's.

The output check has two parts, both on every element the oracle computed:
  * normwise: max |g - o| / max(max |o|, 1e-6) <= 1e-2, the stated tolerance;
  * elementwise: |g - o| <= bound, with the bound derived from the
    arithmetic of a correct float32 evaluation of the epilogue ("Core idea of
    LLM.int8()", step 3: dequantise the int32 result, add the 16-bit outlier
    product; "Class Linear8bitLt", bias).  The int32 accumulator is exact, so
    the only errors are float32 roundings (dequantisation factor and product,
    each addition of the outlier sum, the bias and the final sums), each at
    most 2^-24 of a partial sum no larger than A = |D| + sum |x * w^| + |b|,
    then one rounding to the 16-bit dtype:
        E     = (n_outlier_columns + 8) * 2^-23 * A
        bound = E + u * (|o| + E) + eta
    with u = 2^-11 (fp16) or 2^-8 (bf16) half an ulp relative, and eta half the
    smallest subnormal spacing (2^-25 fp16, 2^-133 bf16).  The factor 2^-23
    (not 2^-24) leaves room for a matrix core that rounds its internal sums
    toward zero.
A dropped or misplaced bias, a dropped outlier term or a wrong dequantisation
factor moves elements far past this bound (tests/test_out_check.py shows it
for every shape the GPU tests use).
"""
import numpy as np

import oracle as O

OUT_TOL = 1e-2
HALF_ULP_REL = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
HALF_SUBNORMAL = {"f16": 2.0 ** -25, "bf16": 2.0 ** -133}


def to_dev(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def normwise_rel(gpu_bits: np.ndarray, ref64: np.ndarray, dtype: str) -> float:
    """max |g - o| / max(max |o|, 1e-6), the output tolerance measure."""
    g = O.decode_bits(gpu_bits, dtype).astype(np.float64)
    den = max(float(np.abs(ref64).max()) if ref64.size else 0.0, 1e-6)
    return float(np.abs(g - ref64).max() / den) if ref64.size else 0.0


def out_bound(r: dict, dtype: str) -> np.ndarray:
    """Per-element bound on |g - o| for a correct float32 epilogue (see above)."""
    E = (r["idx"].size + 8) * 2.0 ** -23 * r["abs64"]
    return E + HALF_ULP_REL[dtype] * (np.abs(r["out64"]) + E) + HALF_SUBNORMAL[dtype]


def out_errors(gpu_bits: np.ndarray, r: dict, dtype: str):
    """(normwise relative error, largest |g - o| / bound over the elements)."""
    if r["out64"].size == 0:
        return 0.0, 0.0
    g = O.decode_bits(gpu_bits, dtype).astype(np.float64).reshape(r["out64"].shape)
    ratio = float((np.abs(g - r["out64"]) / out_bound(r, dtype)).max())
    return normwise_rel(gpu_bits, r["out64"], dtype), ratio


def out_ok(gpu_bits: np.ndarray, r: dict, dtype: str) -> bool:
    nw, ratio = out_errors(gpu_bits, r, dtype)
    return nw <= OUT_TOL and ratio <= 1.0


def assert_out(gpu_bits: np.ndarray, r: dict, dtype: str, what: str = "out"):
    nw, ratio = out_errors(gpu_bits, r, dtype)
    assert nw <= OUT_TOL and ratio <= 1.0, (
        f"{what}: normwise rel err {nw:.3e} (limit {OUT_TOL}), worst element at {ratio:.3f} x its bound")
    return nw, ratio
