"""Seeded synthetic inputs for the LLM.int8() mixed-precision linear.

This module only draws random numbers and stores them in the activation dtype.
It holds none of the method's arithmetic (no threshold test, no absmax, no
rounding to int8, no product), so both the CPU oracle and the GPU path can take
their inputs from it without sharing any computation.

Shapes and value distributions stand in for the workloads the pages discuss:
a 64->64 layer as in the conversion example of "Class Linear8bitLt" (class
docstring), a 16-token decode step and 4096-token prefill steps of 7B- and
175B-class MLP layers as in "Hugging Face integrates LLM.int8() ..." (sections
"Why 8-bit quantization matters", "Empirical evidence"), with a few planted
outlier feature columns of magnitude 6..60, the size class that section "Core
idea of LLM.int8()" singles out.  No model weights or datasets are used.

Rules (one generator per case, numpy PCG64, seed 0 unless given):
  draw order: X base -> outlier column choice -> outlier magnitudes ->
  outlier signs -> W -> bias.
  N(mu, sigma): sigma is the standard deviation.
  "+-U(a,b)": magnitude ~ U(a,b) with an independent fair sign, per element;
  the planted column is replaced in every row.
  fp16 storage: numpy's float32->float16 cast (round to nearest even).
  bf16 storage: float32 bits rounded to the upper 16 bits, nearest even.
Tensors are returned as raw 16-bit patterns (numpy uint16) plus a dtype tag.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclasses.dataclass
class Case:
    name: str
    T: int
    K: int
    N: int
    dtype: str                  # "f16" or "bf16"
    X: np.ndarray               # uint16 bits [T, K]
    W: np.ndarray               # uint16 bits [N, K]
    bias: Optional[np.ndarray]  # uint16 bits [N] or None
    threshold: float
    planted_cols: np.ndarray    # int64, the columns that were replaced
    weights_each_call: bool     # True: W is quantized inside every call

    def sha256(self) -> dict:
        out = {}
        for k in ("X", "W", "bias"):
            a = getattr(self, k)
            if a is not None:
                out[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def _f32_to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F16:
        return a.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = a.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(dtype)


def _draw_activation(rng, T, K, base, n_out, lo, hi, fixed_cols=None, clamp=None):
    if base == "normal":
        x = rng.standard_normal((T, K), dtype=np.float32)
    elif base == "student_t3":
        x = rng.standard_t(3, size=(T, K)).astype(np.float32)
    else:
        raise ValueError(base)
    if clamp is not None:
        np.clip(x, -clamp, clamp, out=x)
    if fixed_cols is not None:
        cols = np.asarray(fixed_cols, dtype=np.int64)
    else:
        cols = np.sort(rng.choice(K, n_out, replace=False)).astype(np.int64)
    mag = rng.uniform(lo, hi, size=(T, cols.size)).astype(np.float32)
    sign = np.where(rng.random((T, cols.size)) < 0.5, -1.0, 1.0).astype(np.float32)
    x[:, cols] = mag * sign
    return x, cols


def _draw_normal(rng, shape, sigma, chunk_rows=2048):
    """N(0, sigma) in float32, drawn row-chunk by row-chunk to bound memory."""
    out = np.empty(shape, dtype=np.float32)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        blk *= np.float32(sigma)
        out[r0:r1] = blk
    return out


def _weight_bits(rng, N, K, sigma, dtype):
    out = np.empty((N, K), dtype=np.uint16)
    for r0 in range(0, N, 2048):
        r1 = min(N, r0 + 2048)
        blk = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        blk *= np.float32(sigma)
        out[r0:r1] = _f32_to_bits(blk, dtype)
    return out


def make_case(name: str, T: int, K: int, N: int, dtype: str = F16, *,
              base: str = "normal", n_out: int = 0, out_lo: float = 6.0,
              out_hi: float = 60.0, fixed_cols=None, clamp=None,
              w_sigma: float = 0.02, bias: Optional[str] = None,
              bias_sigma: float = 0.01, threshold: float = 6.0,
              weights_each_call: bool = False, seed: int = 0) -> Case:
    """Draw one case.  bias: None (no bias), "zero", or "normal"."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x, cols = _draw_activation(rng, T, K, base, n_out, out_lo, out_hi,
                               fixed_cols=fixed_cols, clamp=clamp)
    Xb = _f32_to_bits(x, dtype)
    del x
    Wb = _weight_bits(rng, N, K, w_sigma, dtype)
    if bias is None:
        bb = None
    elif bias == "zero":
        bb = _f32_to_bits(np.zeros(N, np.float32), dtype)
    elif bias == "normal":
        bb = _f32_to_bits(rng.standard_normal(N, dtype=np.float32) * np.float32(bias_sigma), dtype)
    else:
        raise ValueError(bias)
    return Case(name, T, K, N, dtype, Xb, Wb, bb, float(threshold), cols,
                weights_each_call)


# The workloads: the pages' five, a 64-token decode batch, and the
# clamped-base variant of the stress case.
CONFIGS = {
    # 64->64 layer with bias, two planted outlier columns.
    "tiny": dict(T=8, K=64, N=64, dtype=F16, fixed_cols=[3, 17], out_lo=8.0,
                 out_hi=20.0, w_sigma=0.02, bias="normal"),
    # 16-token decode step of a 4096->4096 projection; weights pre-quantized.
    "decode": dict(T=16, K=4096, N=4096, dtype=F16, n_out=6, w_sigma=0.02,
                   bias="zero"),
    # The same projection for a batch of 64 tokens: past the fused one-launch
    # path, on the weight-streaming GEMM (a small-batch serving step).
    "decode_b64": dict(T=64, K=4096, N=4096, dtype=F16, n_out=6, w_sigma=0.02,
                       bias="zero"),
    # 4096-token prefill through a 7B-class MLP up-projection.
    "prefill_mlp_up": dict(T=4096, K=4096, N=11008, dtype=F16, n_out=4,
                           w_sigma=0.02),
    # 4096-token prefill through a 175B-class FFN up-projection.
    "ffn_175b": dict(T=4096, K=12288, N=49152, dtype=F16, n_out=12,
                     w_sigma=0.01),
    # bf16, heavy-tailed Student-t(3) activations, weights quantized each call.
    "stress_bf16": dict(T=2048, K=8192, N=28672, dtype=BF16, base="student_t3",
                        n_out=82, out_hi=100.0, w_sigma=0.02,
                        weights_each_call=True),
    # As stress_bf16 with the t(3) base clipped to +-5.9: exactly 82 outliers.
    "stress_bf16_clamped": dict(T=2048, K=8192, N=28672, dtype=BF16,
                                base="student_t3", clamp=5.9, n_out=82,
                                out_hi=100.0, w_sigma=0.02,
                                weights_each_call=True),
}

CONFIG_ORDER = ["tiny", "decode", "decode_b64", "prefill_mlp_up", "ffn_175b",
                "stress_bf16", "stress_bf16_clamped"]


def config_case(name: str, seed: int = 0) -> Case:
    return make_case(name, seed=seed, **CONFIGS[name])


def random_case(T, K, N, dtype=F16, seed=0, n_out=3, bias="normal",
                threshold=6.0, out_lo=6.0, out_hi=60.0, bias_sigma=0.5) -> Case:
    """A small case of arbitrary shape for parity sweeps.  The bias is drawn
    N(0, 0.5), the size of a typical output element (N(0, 1) activations
    times N(0, 0.02) weights summed over a few hundred to a few thousand
    features), so that a lost or misplaced bias term shows in every output."""
    n_out = min(n_out, K)
    return make_case(f"rand_{T}x{K}x{N}_{dtype}_{seed}", T, K, N, dtype,
                     n_out=n_out, out_lo=out_lo, out_hi=out_hi, bias=bias,
                     bias_sigma=bias_sigma, threshold=threshold, seed=seed)


def matrix_bits(R: int, C: int, dtype: str = F16, seed: int = 0) -> np.ndarray:
    """A 16-bit matrix [R, C] (raw bits) with rows of varied range: each row
    N(0, 1) times a row scale U(0.01, 30) plus a row offset U(-5, 5); every
    7th row made non-negative, every 9th (from 1) non-positive, every 11th
    (from 2) all zero, column 3 (when present) exactly zero."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((R, C), dtype=np.float32)
    x *= rng.uniform(0.01, 30.0, size=(R, 1)).astype(np.float32)
    x += rng.uniform(-5.0, 5.0, size=(R, 1)).astype(np.float32)
    x[::7] = np.abs(x[::7])
    x[1::9] = -np.abs(x[1::9])
    x[2::11] = 0.0
    if C > 3:
        x[:, 3] = 0.0
    return _f32_to_bits(x, dtype)
