"""CPU oracle for the LLM.int8() mixed-precision decomposition linear (forward).

TEST INFRASTRUCTURE.  This module is the slow, plain reference the GPU path is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path never does.  It shares no code
with the HIP library: it reads raw 16-bit inputs and does every step itself in
NumPy (float32 where a quantised code is decided, float64 elsewhere).

What it computes, with the passage each step follows:

  O1  X[T,K] in fp16/bf16, widened to float32 (exact).
  O2  Outlier feature columns: column c is an outlier when some row has
      |X[t,c]| > threshold ("Class Linear8bitLt", __init__ Args, threshold;
      "Hugging Face integrates LLM.int8() ...", section "Core idea of
      LLM.int8()", step 1; inference-research record "LLM.int8() /
      bitsandbytes int8", field "Activation scheme": outlier feature
      dimensions, not outlier values or tokens).  idx is ascending
      (the issue "How to get the information of which columns have been
      quantified?" prints state.idx in ascending order).
  O3-O5  Vector-wise absmax quantisation of the remaining activations, one
      scale per row ("Core idea", step 2: row-wise for activations; section
      "Quantization mechanics": divide by the absolute maximum, scale to 127,
      round, range [-127, 127]).
  O6  The same per output row of W[N,K] ("Core idea", step 2: column-wise for
      the weight in X.W orientation, i.e. per row of nn.Linear's [out, in]
      weight), giving CB and SCB ("Integration into transformers": int8 values
      in [-127, 127], recovery (CB * SCB) / 127).
  O7  int8 x int8 products summed exactly (int32 range).
  O8  Dequantisation acc * SCA * SCB / 127^2 ("Core idea", step 3).
  O9  Recovered weight for the outlier columns, (CB * SCB) / 127 in float32,
      rounded to the activation dtype ("Integration into transformers").
  O10 The 16-bit outlier product X[:, idx] . W^[:, idx]^T ("Core idea", step 2:
      outliers multiplied in 16-bit; record field "Activation scheme": a
      second 16-bit matrix multiplication).
  O11 out = D + O + bias, rounded once to the activation dtype ("Core idea",
      step 3: dequantise and sum with the outlier result).

Readings where the pages leave a step open (each one is listed, with its
reason, in the design notes of the repository):
  * "exceeds" is strict (>), compared between exact float32 values, with the
    threshold first converted to float32.
  * threshold <= 0 (the constructor default 0.0) turns the decomposition off:
    no outlier columns.  A NaN threshold is an error.
  * Whole outlier columns are excluded from the row absmax and set to 0 in CA.
  * Scale factor s = fl32(127 / absmax), code = round_half_away(fl32(x * s)),
    clamped to [-127, 127].  A row whose absmax is 0 gets SCA = 0 and CA = 0.
    For an absmax below 2^-100 (bf16 only: an fp16 absmax is at least 2^-24)
    127 / absmax can overflow float32; there x and the absmax are scaled by
    2^64 first (exact), which gives the plain form's codes wherever that form
    is finite.
  * SCA and SCB store the absmax itself, as float32.
  * The outlier product uses X unquantised and the recovered weight rounded to
    the activation dtype, in both weight modes.

Vector-wise quantisation on its own (not a step of the forward; section
"Quantization mechanics": zero-point and absmax, each row-wise or
column-wise):
  V1  absmax per row or per column: the O3-O5 quantiser without exclusions,
      applied to X or to X transposed; the scale stored is the absmax.
  V2  zero-point per row or per column.  Readings: the range is the vector's
      [min, max] widened to contain 0 (so 0.0 has an exact code, the zero
      point); nd = fl32(254 / fl32(hi - lo)); zp = round_half_away(fl32(-lo *
      nd)) - 127, an integer in [-127, 127]; code = clamp(round_half_away(
      fl32(x * nd)) + zp, -127, 127).  For [-1, 1] this is absmax with scale
      127.  An all-zero vector gets nd = 0, zp = 0 and codes 0.  Stored: nd
      (float32) and zp (int32); x is recovered as (code - zp) / nd.

Parity pins: every step above is pinned by CPU tests (worked example, closed
forms, brute force, invariants), the output included (the all-outlier case
equals the plain product, the integer case the textbook matmul, and every
output lies within the a-priori error bound).  The output is the exact fp64
value of the epilogue; a 16-bit output computed with fp32 sums in another
order is equally correct, so the GPU path's output is compared with it within
a tolerance and an elementwise bound, not bit for bit.
"""
from __future__ import annotations

import numpy as np

F16 = "f16"
BF16 = "bf16"
INT8_MAX = 127
TINY_ABSMAX = np.float32(2.0 ** -100)  # absmax below this: the row is scaled by PRESCALE first
PRESCALE = np.float32(2.0 ** 64)


# ---------------------------------------------------------------- dtypes ----

def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw fp16/bf16 bit patterns -> float32 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _round_to_bf16_value(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and float32's exponent range, so the
    quantum at x = m * 2**e (0.5 <= |m| < 1) is 2**(e-8), and never finer than
    the subnormal spacing 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def round_to_dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32/float64 values -> bits of the nearest fp16/bf16 (ties to even)."""
    x = np.asarray(x)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        v = _round_to_bf16_value(x.astype(np.float64)).astype(np.float32)
        return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------ O2: outliers ----

def outlier_columns(X: np.ndarray, threshold: float) -> np.ndarray:
    """Ascending int32 indices of the columns where some |X[t, c]| > threshold.

    X: float32 [T, K].  threshold <= 0 (the module default) gives no columns;
    NaN is rejected.
    """
    if np.isnan(threshold):
        raise ValueError("threshold is NaN")
    tau = np.float32(threshold)
    if not tau > 0:
        return np.zeros(0, dtype=np.int32)
    if X.shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    col_max = np.max(np.abs(X), axis=0)
    return np.nonzero(col_max > tau)[0].astype(np.int32)


def outlier_bitmap(idx: np.ndarray, K: int) -> np.ndarray:
    """The outlier set as uint32 words: bit (c % 32) of word c // 32 is set for c in idx.

    (An encoding of O2's set for the library's interface; the pages only name
    the set, state.idx.)
    """
    words = np.zeros((K + 31) // 32, dtype=np.uint64)
    idx = np.asarray(idx, dtype=np.int64)
    np.bitwise_or.at(words, idx // 32, np.uint64(1) << (idx % 32).astype(np.uint64))
    return words.astype(np.uint32)


# ---------------------------------------------- O3-O6: absmax quantisation ----

def round_half_away(v: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, halves away from zero, evaluated exactly.

    v holds float32 values of magnitude <= 128; in float64, |v| + 0.5 is exact,
    so floor() sees the true sum (unlike float32, where 0.49999997 + 0.5 rounds
    up to 1.0).
    """
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def absmax_quantize_rows(X: np.ndarray, excluded_cols=None):
    """Row-wise absmax quantisation to int8 in [-127, 127].

    X: float32 [R, C].  Columns in excluded_cols are left out of the absmax and
    coded 0.  Returns (codes int8 [R, C], absmax float32 [R]).
    """
    X = np.asarray(X, dtype=np.float32)
    Xr = X.copy()
    if excluded_cols is not None and len(excluded_cols):
        Xr[:, np.asarray(excluded_cols, dtype=np.int64)] = 0
    amax = np.max(np.abs(Xr), axis=1) if Xr.shape[1] else np.zeros(Xr.shape[0], np.float32)
    amax = amax.astype(np.float32)
    codes = np.zeros(Xr.shape, dtype=np.int8)
    live = amax > 0
    if np.any(live):
        # Below 2^-100 (bf16 rows only) the absmax and the row are taken
        # 2^64 larger first, exactly, so that 127 / absmax stays finite;
        # wherever the plain factor is finite this changes no code.
        a = amax[live]
        pre = np.where(a < TINY_ABSMAX, PRESCALE, np.float32(1)).astype(np.float32)
        s = np.float32(INT8_MAX) / (a * pre)               # fl32(127 / absmax)
        v = (Xr[live] * pre[:, None]) * s[:, None]         # fl32(x * s)
        assert v.dtype == np.float32
        q = np.clip(round_half_away(v), -INT8_MAX, INT8_MAX)
        codes[live] = q.astype(np.int8)
    return codes, amax


def quantize_activations(X: np.ndarray, threshold: float):
    """O2-O5: (idx, CA, SCA) for float32 activations X [T, K]."""
    idx = outlier_columns(X, threshold)
    CA, SCA = absmax_quantize_rows(X, idx)
    return idx, CA, SCA


def quantize_weight(W: np.ndarray):
    """O6: (CB int8 [N, K], SCB float32 [N]) for float32 weights W [N, K]."""
    return absmax_quantize_rows(W, None)


# ------------------------------- V1-V2: vector-wise quantisation variants ----

def absmax_quantize(X: np.ndarray, axis: int):
    """V1: absmax codes with one scale per row (axis=1) or per column (axis=0).
    Returns (codes int8 like X, absmax float32 [rows or columns])."""
    X = np.asarray(X, dtype=np.float32)
    if axis == 1:
        return absmax_quantize_rows(X, None)
    codes, amax = absmax_quantize_rows(X.T, None)
    return np.ascontiguousarray(codes.T), amax


def zeropoint_quantize_rows(X: np.ndarray):
    """V2 per row: (codes int8 [R, C], nd float32 [R], zp int32 [R])."""
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    if C == 0:
        return np.zeros((R, 0), np.int8), np.zeros(R, np.float32), np.zeros(R, np.int32)
    lo = np.minimum(X.min(axis=1), np.float32(0)).astype(np.float32)
    hi = np.maximum(X.max(axis=1), np.float32(0)).astype(np.float32)
    width = (hi - lo).astype(np.float32)                    # fl32(hi - lo)
    nd = np.zeros(R, dtype=np.float32)
    zp = np.zeros(R, dtype=np.int32)
    codes = np.zeros((R, C), dtype=np.int8)
    live = width > 0
    if np.any(live):
        nd[live] = np.float32(254) / width[live]              # fl32(254 / width)
        zl = (-lo[live] * nd[live]).astype(np.float32)        # fl32(-lo * nd)
        zp[live] = (round_half_away(zl) - 127).astype(np.int32)
        v = X[live] * nd[live][:, None]                        # fl32(x * nd)
        assert v.dtype == np.float32
        q = np.clip(round_half_away(v) + zp[live][:, None], -INT8_MAX, INT8_MAX)
        codes[live] = q.astype(np.int8)
    return codes, nd, zp


def zeropoint_quantize(X: np.ndarray, axis: int):
    """V2 per row (axis=1) or per column (axis=0)."""
    X = np.asarray(X, dtype=np.float32)
    if axis == 1:
        return zeropoint_quantize_rows(X)
    codes, nd, zp = zeropoint_quantize_rows(X.T)
    return np.ascontiguousarray(codes.T), nd, zp


def zeropoint_dequantize(codes: np.ndarray, nd: np.ndarray, zp: np.ndarray, axis: int) -> np.ndarray:
    """x^ = (code - zp) / nd (float64); 0 where nd = 0."""
    n = nd.astype(np.float64)
    inv = np.divide(1.0, n, out=np.zeros_like(n), where=n > 0)
    z = zp.astype(np.float64)
    if axis == 1:
        return (codes.astype(np.float64) - z[:, None]) * inv[:, None]
    return (codes.astype(np.float64) - z[None, :]) * inv[None, :]


# --------------------------------------------------- O7: int8 accumulation ----

def int8_accumulate(CA: np.ndarray, CB: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """acc[t, n] = sum_k CA[t, k] * CB[n, k], exactly, as int32.

    Every product is an integer of magnitude <= 127^2 and every partial sum
    stays far below 2^53, so a float64 matrix product is exact in any order.
    """
    A = CA.astype(np.float64)
    out = np.empty((CA.shape[0], CB.shape[0]), dtype=np.int64)
    for n0 in range(0, CB.shape[0], chunk):
        n1 = min(CB.shape[0], n0 + chunk)
        out[:, n0:n1] = np.rint(A @ CB[n0:n1].astype(np.float64).T).astype(np.int64)
    if out.size:
        assert np.abs(out).max() < 2 ** 31, "int32 accumulator overflow"
    return out.astype(np.int32)


# ------------------------------------------------------------ O8-O11: out ----

def dequantize(acc: np.ndarray, SCA: np.ndarray, SCB: np.ndarray) -> np.ndarray:
    """O8: acc * SCA[t] * SCB[n] / 127^2 in float64."""
    return (acc.astype(np.float64) * SCA.astype(np.float64)[:, None]
            * SCB.astype(np.float64)[None, :]) / float(INT8_MAX * INT8_MAX)


def recover_weight(CB_cols: np.ndarray, SCB: np.ndarray, dtype: str) -> np.ndarray:
    """O9: values of dtype( fl32( fl32(CB * SCB) / 127 ) ), as float64."""
    prod = CB_cols.astype(np.float32) * SCB.astype(np.float32)[:, None]
    rec = prod / np.float32(INT8_MAX)
    assert rec.dtype == np.float32
    return decode_bits(round_to_dtype_bits(rec, dtype), dtype).astype(np.float64)


def linear_forward(X_bits, dtype, CB, SCB, bias_bits, threshold, rows=None, cols=None):
    """The whole forward, O1-O11.

    X_bits uint16 [T, K]; CB int8 [N, K]; SCB float32 [N]; bias_bits uint16
    [N] or None.  rows / cols optionally select the output rows and columns to
    evaluate (the outlier set is always taken over every row of X).

    Returns a dict: idx, CA, SCA (selected rows), acc (selected block, int32),
    out64 (float64, before the final rounding), out_bits (uint16), and abs64 =
    |D| + sum over outlier columns of |X[t, c] * W^[n, c]| + |bias[n]| (float64),
    the magnitude that bounds the rounding error of any float32 evaluation of
    O8-O11.
    """
    X = decode_bits(X_bits, dtype)
    idx = outlier_columns(X, threshold)
    Xs = X if rows is None else X[np.asarray(rows)]
    CBs = CB if cols is None else CB[np.asarray(cols)]
    SCBs = SCB if cols is None else SCB[np.asarray(cols)]
    CA, SCA = absmax_quantize_rows(Xs, idx)
    acc = int8_accumulate(CA, CBs)
    D = dequantize(acc, SCA, SCBs)
    abs64 = np.abs(D)
    if idx.size:
        What = recover_weight(CBs[:, idx], SCBs, dtype)
        Xo = Xs[:, idx].astype(np.float64)
        O = Xo @ What.T
        abs64 += np.abs(Xo) @ np.abs(What).T
    else:
        O = np.zeros_like(D)
    out64 = D + O
    if bias_bits is not None:
        b = decode_bits(bias_bits, dtype).astype(np.float64)
        b = (b if cols is None else b[np.asarray(cols)])[None, :]
        out64 = out64 + b
        abs64 += np.abs(b)
    return dict(idx=idx, CA=CA, SCA=SCA, acc=acc, out64=out64, abs64=abs64,
                out_bits=round_to_dtype_bits(out64, dtype))


def quantize_weight_bits(W_bits, dtype, rows=None):
    """O6 on raw fp16/bf16 weight bits (optionally a subset of rows)."""
    W = decode_bits(W_bits if rows is None else W_bits[np.asarray(rows)], dtype)
    return quantize_weight(W)
