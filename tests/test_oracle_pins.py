"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Each test names the passage or closed form it checks.  None of them compares
the oracle with itself: the expected values come from the pages' worked
example and repro, from hand derivations, from brute-force loops, from
textbook special cases or from a priori error bounds.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import config_case, random_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- P-1 -----
def test_absmax_worked_example_fp32():
    """Quantization mechanics (absmax bullet): scale 127/5.4 ~ 23.5, codes in [-127, 127]."""
    g = _load("absmax_worked_example.json")
    x = np.array([g["vector"]], np.float32)
    codes, amax = O.absmax_quantize_rows(x)
    assert amax[0] == np.float32(g["absmax"])
    scale = np.float32(127) / amax[0]
    assert abs(float(scale) - g["scale_printed"]) <= g["scale_printed_resolution"]
    lo, hi = g["code_range"]
    assert codes.min() >= lo and codes.max() <= hi
    assert codes[0].tolist() == g["codes_derived"]


def test_absmax_worked_example_fp16():
    """Same example after rounding the vector to fp16 (5.4 -> 5.3984375): same codes."""
    g = _load("absmax_worked_example.json")
    x = O.decode_bits(_f16([g["vector"]]), "f16")
    codes, amax = O.absmax_quantize_rows(x)
    assert amax[0] == np.float32(5.3984375)
    assert codes[0].tolist() == g["codes_derived"]


def test_weight_bits_worked_example_and_row_selection():
    """The weight quantiser on raw 16-bit patterns: the worked example's vector
    as a weight row gives the page's codes and its fp16 absmax, and a row
    subset gives exactly those rows of the whole weight's codes and scales."""
    g = _load("absmax_worked_example.json")
    W = np.stack([_f16([g["vector"]])[0], _f16([[-v for v in g["vector"]]])[0]])
    CB, SCB = O.quantize_weight_bits(W, "f16")
    assert CB[0].tolist() == g["codes_derived"]
    assert CB[1].tolist() == [-c for c in g["codes_derived"]]
    assert SCB.tolist() == [np.float32(5.3984375)] * 2
    case = random_case(7, 40, 13, dtype="bf16", seed=5, n_out=0)
    CBf, SCBf = O.quantize_weight_bits(case.W, "bf16")
    assert np.isfinite(SCBf).all() and (SCBf > 0).all()
    rows = [12, 0, 6]
    CBr, SCBr = O.quantize_weight_bits(case.W, "bf16", rows=rows)
    assert np.array_equal(CBr, CBf[rows]) and np.array_equal(SCBr, SCBf[rows])


@pytest.mark.parametrize("k", [90, 100, 118, 122, 124])
def test_tiny_rows_keep_their_codes(k):
    """Scaling a row by a power of two (exactly) leaves its codes unchanged and
    scales its absmax, also where the absmax falls below 2^-100 and 127 /
    absmax would overflow float32 (k >= 122 here): the quantiser scales such
    a row and its absmax by 2^64 first.  bf16 rows with magnitudes in
    [2^-4, 4], so 2^-k times them stays a normal (exact) bf16 value."""
    rng = np.random.default_rng(k)
    mag = np.exp2(rng.uniform(-4, 2, size=(6, 40)))
    X = O.decode_bits(O.round_to_dtype_bits(mag * rng.choice([-1.0, 1.0], size=mag.shape), "bf16"), "bf16")
    X[1, ::3] = 0.0                                    # zeros in a row
    codes, amax = O.absmax_quantize_rows(X)
    scaled = (X.astype(np.float64) * 2.0 ** -k).astype(np.float32)
    assert np.array_equal(scaled.astype(np.float64) * 2.0 ** k, X.astype(np.float64))  # exact
    codes2, amax2 = O.absmax_quantize_rows(scaled)
    assert np.array_equal(codes2, codes)
    assert np.array_equal(amax2.astype(np.float64), amax.astype(np.float64) * 2.0 ** -k)
    assert (np.abs(codes).max(axis=1) == 127).all()


def test_subnormal_rows_code_like_their_scaled_copies():
    """Rows of bf16 subnormals (absmax down to 2^-133): their codes equal those
    of the same rows scaled up by 2^64, which is exact and lands in the normal
    range, and the row maximum gets code 127."""
    rng = np.random.default_rng(5)
    bits = rng.integers(1, 0x80, size=(5, 24), dtype=np.uint16)      # bf16 subnormals
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)  # either sign
    bits[0] = 0x0001                                                  # every value the smallest subnormal
    bits[1, 5:] = 0                                                   # zeros beside them
    X = O.decode_bits(bits, "bf16")
    assert (np.abs(X) < 2.0 ** -126).all()
    codes, amax = O.absmax_quantize_rows(X)
    big = (X.astype(np.float64) * 2.0 ** 64).astype(np.float32)
    codes2, _ = O.absmax_quantize_rows(big)
    assert np.array_equal(codes, codes2)
    assert (np.abs(codes).max(axis=1) == 127).all()
    assert np.array_equal(codes[0], np.where(X[0] > 0, 127, -127).astype(np.int8))


# ---------------------------------------------------------------- P-2 -----
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_weight_recovery_bound(dtype):
    """Integration into transformers: (CB * SCB) / 127 gives back W to half a step."""
    case = random_case(4, 96, 33, dtype=dtype, seed=5)
    W = O.decode_bits(case.W, dtype)
    CB, SCB = O.quantize_weight(W)
    assert CB.min() >= -127 and CB.max() <= 127
    rec32 = (CB.astype(np.float32) * SCB[:, None]) / np.float32(127)
    err = np.abs(rec32.astype(np.float64) - W)
    bound = SCB.astype(np.float64)[:, None] * (1 / 254 + 2.0 ** -21)
    assert np.all(err <= bound)
    # after rounding to the activation dtype, half an ulp more
    What = O.recover_weight(CB, SCB, dtype)
    u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
    err2 = np.abs(What - W)
    assert np.all(err2 <= bound + np.abs(What) * u + 2.0 ** -25)
    # each row's largest magnitude maps to +-127
    assert np.all(np.abs(CB).max(axis=1) == 127)


def _fl32(q):
    """Exact rational -> the nearest float32 value (ties to even), as a Fraction."""
    from fractions import Fraction
    if q == 0:
        return Fraction(0)
    sgn = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormal spacing below 2^-126
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * ulp


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_weight_recovery_rounding_order_exact(dtype):
    """The Hugging Face integration page ("Integration into transformers")
    writes the recovery as (CB * SCB) / 127, read literally: the product
    first, then the division, each rounded to float32, then one rounding to
    the 16-bit dtype.  Exact rational arithmetic with explicit
    round-to-nearest-even reproduces recover_weight bit for bit, and the pin
    has teeth: on these inputs dividing the scale first
    (CB * fl32(SCB / 127)) gives different float32 values."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    SCB = (rng.uniform(0.01, 3.0, size=64) * rng.choice([1e-3, 1.0, 1e3], size=64)).astype(np.float32)
    CB = rng.integers(-127, 128, size=(64, 16)).astype(np.int8)
    got = O.recover_weight(CB, SCB, dtype)
    differs = 0
    for n in range(64):
        s = Fraction(float(SCB[n]))
        for k in range(16):
            c = int(CB[n, k])
            v = _fl32(_fl32(c * s) / 127)
            ref16 = O.decode_bits(O.round_to_dtype_bits(np.float64(v), dtype), dtype)
            assert got[n, k] == float(ref16), (n, k)
            differs += v != _fl32(c * _fl32(s / 127))
    assert differs > 0
    # a scale of 127 * 2^j recovers the codes exactly scaled by 2^j
    for j in (-6, 0, 5):
        sc = np.full(4, np.float32(127.0 * 2.0 ** j))
        cb = np.array([[-127, -1, 0, 1, 64, 127]] * 4, dtype=np.int8)
        np.testing.assert_array_equal(O.recover_weight(cb, sc, dtype), cb.astype(np.float64) * 2.0 ** j)


# ---------------------------------------------------------------- P-3 -----
def test_threshold_zero_is_no_decomposition():
    """Class Linear8bitLt: threshold defaults to 0.0 and the plain int8 examples use no
    outlier split; threshold <= 0 therefore gives no outlier columns, the same result
    as an infinite threshold, and the output is the int8 part alone."""
    case = random_case(6, 40, 9, seed=3, n_out=2)
    W = O.decode_bits(case.W, "f16")
    CB, SCB = O.quantize_weight(W)
    r0 = O.linear_forward(case.X, "f16", CB, SCB, case.bias, 0.0)
    rneg = O.linear_forward(case.X, "f16", CB, SCB, case.bias, -1.0)
    rinf = O.linear_forward(case.X, "f16", CB, SCB, case.bias, float("inf"))
    assert r0["idx"].size == 0 and rneg["idx"].size == 0 and rinf["idx"].size == 0
    for k in ("CA", "SCA", "acc", "out_bits"):
        assert np.array_equal(r0[k], rinf[k]) and np.array_equal(r0[k], rneg[k])
    # SCA is the plain row absmax over every column
    X = O.decode_bits(case.X, "f16")
    assert np.array_equal(r0["SCA"], np.abs(X).max(axis=1))
    with pytest.raises(ValueError):
        O.outlier_columns(X, float("nan"))


# ---------------------------------------------------------------- P-4 -----
def test_issue_tiny_threshold_flags_every_column():
    """Issue 1609: threshold 0.1 on x[2, 8] ~ N(0,1) flags all 8 columns, so
    state.idx = [0..7], nothing is left for int8 and the layer is a plain 16-bit
    product with the recovered weight."""
    g = _load("issue_all_columns_flagged.json")
    T, K = g["x_shape"]
    N = g["out_features"]
    rng = np.random.default_rng(1609)
    x = rng.standard_normal((T, K)).astype(np.float32)
    # brute force: this draw does have, in each column, a value above 0.1
    for c in range(K):
        assert any(abs(float(x[t, c])) > g["threshold"] for t in range(T))
    Xb = _f16(x)
    W = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.3)
    Wb = _f16(W)
    bias = _f16(rng.standard_normal(N) * 0.1)
    CB, SCB = O.quantize_weight(O.decode_bits(Wb, "f16"))
    r = O.linear_forward(Xb, "f16", CB, SCB, bias, g["threshold"])
    assert r["idx"].tolist() == g["state_idx_printed"]
    assert not r["CA"].any() and not r["SCA"].any() and not r["acc"].any()
    # out = X . What^T + b through a library matrix product
    What = O.recover_weight(CB, SCB, "f16")
    ref = O.decode_bits(Xb, "f16").astype(np.float64) @ What.T + O.decode_bits(bias, "f16")
    assert np.allclose(r["out64"], ref, rtol=0, atol=1e-12)
    assert np.array_equal(r["out_bits"], ref.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------- P-5 -----
@settings(max_examples=25, deadline=None)
@given(T=st.integers(1, 9), K=st.integers(1, 17), N=st.integers(1, 9),
       seed=st.integers(0, 10 ** 6), tau=st.sampled_from([0.0, 0.5, 1.5, 6.0]))
def test_brute_force_idx_and_accumulators(T, K, N, seed, tau):
    """Definition: idx by a column-by-column scan; acc by integer triple loops."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * 2).astype(np.float32)
    X = O.decode_bits(_f16(x), "f16")
    idx = O.outlier_columns(X, tau)
    brute = [c for c in range(K) if tau > 0 and max(abs(float(X[t, c])) for t in range(T)) > tau]
    assert idx.tolist() == brute
    CA = rng.integers(-127, 128, size=(T, K)).astype(np.int8)
    CB = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    acc = O.int8_accumulate(CA, CB)
    for t in range(T):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(CA[t, k]) * int(CB[n, k])
            assert int(acc[t, n]) == s


def test_accumulator_extremes_exact():
    """All +-127 operands at K = 133144 reach 2147117104 < 2^31 - 1 exactly."""
    K = 133144
    CA = np.full((1, K), 127, np.int8)
    CB = np.full((2, K), 127, np.int8)
    CB[1] = -127
    acc = O.int8_accumulate(CA, CB)
    assert acc.tolist() == [[127 * 127 * K, -127 * 127 * K]]


# ---------------------------------------------------------------- P-6 -----
def test_integer_special_case_is_textbook_matmul():
    """X and W integer valued in [-127, 127], each row reaching 127: the scale is
    exactly 1, so CA = X, CB = W and acc is the integer matrix product."""
    rng = np.random.default_rng(6)
    T, K, N = 5, 23, 7
    Xi = rng.integers(-126, 127, size=(T, K))
    Wi = rng.integers(-126, 127, size=(N, K))
    Xi[np.arange(T), rng.integers(0, K, T)] = 127
    Wi[np.arange(N), rng.integers(0, K, N)] = -127
    X = O.decode_bits(_f16(Xi), "f16")
    W = O.decode_bits(_f16(Wi), "f16")
    idx, CA, SCA = O.quantize_activations(X, 1000.0)
    CB, SCB = O.quantize_weight(W)
    assert idx.size == 0
    assert np.array_equal(CA, Xi) and np.array_equal(CB, Wi)
    assert np.all(SCA == 127) and np.all(SCB == 127)
    acc = O.int8_accumulate(CA, CB)
    assert np.array_equal(acc.astype(np.int64), Xi @ Wi.T)
    # dequantisation with SCA = SCB = 127 is the identity on acc
    assert np.array_equal(O.dequantize(acc, SCA, SCB), (Xi @ Wi.T).astype(np.float64))


# ---------------------------------------------------------------- P-7 -----
def test_rounding_is_half_away_from_zero():
    """Halves round away from zero (half-even would give [127, 2, -2, 0, 2, 0])."""
    X = O.decode_bits(_f16([[127, 2.5, -2.5, 0.5, 1.5, -0.5]]), "f16")
    codes, amax = O.absmax_quantize_rows(X)
    assert amax[0] == 127
    assert codes[0].tolist() == [127, 3, -3, 1, 2, -1]


def test_round_half_away_float32_trap():
    """0.49999997 (the float32 below 1/2) must round to 0, not to 1."""
    v = np.array([np.nextafter(np.float32(0.5), np.float32(0)), -np.nextafter(np.float32(0.5), np.float32(0)),
                  0.5, -0.5, 126.5, -126.5, 127.0], np.float32)
    assert O.round_half_away(v).tolist() == [0, 0, 1, -1, 127, -127, 127]


# ---------------------------------------------------------------- P-8 -----
def test_threshold_is_strict():
    """'exceeds': a column whose largest magnitude is exactly 6.0 is not an outlier;
    one at the next fp16 value, 6.00390625, is."""
    x = np.zeros((3, 4), np.float32)
    x[1, 0] = 6.0
    x[2, 1] = -6.0
    x[0, 2] = 6.00390625
    x[1, 3] = -6.00390625
    X = O.decode_bits(_f16(x), "f16")
    assert O.outlier_columns(X, 6.0).tolist() == [2, 3]


# ---------------------------------------------------------------- P-9 -----
@settings(max_examples=30, deadline=None)
@given(T=st.integers(1, 12), K=st.integers(1, 40), seed=st.integers(0, 10 ** 6),
       tau=st.sampled_from([0.0, 1.0, 2.5, 6.0]))
def test_quantizer_invariants(T, K, seed, tau):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * 3).astype(np.float32)
    X = O.decode_bits(_f16(x), "f16")
    idx, CA, SCA = O.quantize_activations(X, tau)
    assert CA.min() >= -127 and CA.max() <= 127
    assert not CA[:, idx].any()
    for t in range(T):
        if SCA[t] > 0:
            assert np.abs(CA[t]).max() == 127
        else:
            assert not CA[t].any()
    # odd symmetry
    idx2, CA2, SCA2 = O.quantize_activations(-X, tau)
    assert np.array_equal(idx2, idx) and np.array_equal(CA2, -CA) and np.array_equal(SCA2, SCA)
    # column permutation equivariance
    p = rng.permutation(K)
    idx3, CA3, SCA3 = O.quantize_activations(X[:, p], tau)
    assert sorted(p[idx3].tolist()) == idx.tolist()
    assert np.array_equal(CA3, CA[:, p]) and np.array_equal(SCA3, SCA)
    # monotone in the threshold
    if tau > 0:
        idx4 = O.outlier_columns(X, tau * 2)
        assert set(idx4.tolist()) <= set(idx.tolist())


@settings(max_examples=20, deadline=None)
@given(T=st.integers(1, 6), K=st.integers(1, 24), seed=st.integers(0, 10 ** 6), j=st.integers(-4, 4))
def test_power_of_two_scaling(T, K, seed, j):
    """With no outliers, scaling X by 2^j leaves CA unchanged and scales SCA by 2^j."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    X = O.decode_bits(_f16(x), "f16")
    _, CA, SCA = O.quantize_activations(X, 0.0)
    _, CA2, SCA2 = O.quantize_activations(X * np.float32(2.0 ** j), 0.0)
    assert np.array_equal(CA, CA2)
    assert np.array_equal(SCA2, SCA * np.float32(2.0 ** j))


def _apriori_bound(X, W, idx, SCA, SCB, What, dtype):
    keep = np.ones(X.shape[1], bool)
    keep[idx] = False
    X64, W64 = X.astype(np.float64), W.astype(np.float64)
    dX = (SCA.astype(np.float64) * (1 / 254 + 2.0 ** -21))[:, None]   # per row
    dW = (SCB.astype(np.float64) * (1 / 254 + 2.0 ** -21))[:, None]   # per weight row
    Xk, Wk = np.abs(X64[:, keep]), np.abs(W64[:, keep])
    b = (dX * Wk.sum(1)[None, :] + Xk @ np.broadcast_to(dW, Wk.shape).T
         + dX * dW.T * keep.sum())
    if idx.size:
        u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
        dWo = dW + np.abs(What) * u + 2.0 ** -24
        b = b + np.abs(X64[:, idx]) @ np.broadcast_to(dWo, (W.shape[0], idx.size)).T
    return b * (1 + 1e-9) + 1e-12


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_output_within_apriori_error_bound(dtype, seed):
    """|out - (X W^T + b)| obeys the error bound that follows from half-step
    quantisation of both operands on the int8 part and the recovered weight on the
    outlier part.  A dropped outlier term, a wrong scale or a transposed operand
    breaks it."""
    case = random_case(7, 70, 13, dtype=dtype, seed=seed, n_out=3)
    X = O.decode_bits(case.X, dtype)
    W = O.decode_bits(case.W, dtype)
    bias = O.decode_bits(case.bias, dtype).astype(np.float64) * 50.0
    bias_bits = O.round_to_dtype_bits(bias, dtype)
    bias = O.decode_bits(bias_bits, dtype).astype(np.float64)
    CB, SCB = O.quantize_weight(W)
    r = O.linear_forward(case.X, dtype, CB, SCB, bias_bits, case.threshold)
    assert r["idx"].tolist() == sorted(case.planted_cols.tolist())
    What = O.recover_weight(CB[:, r["idx"]], SCB, dtype)
    exact = X.astype(np.float64) @ W.astype(np.float64).T + bias[None, :]
    bound = _apriori_bound(X, W, r["idx"], r["SCA"], SCB, What, dtype)
    assert np.all(np.abs(r["out64"] - exact) <= bound)
    # and the outlier columns matter: without them the error is far beyond the bound
    no_out = r["out64"] - X[:, r["idx"]].astype(np.float64) @ What.T
    assert np.any(np.abs(no_out - exact) > bound)


def test_tiny_config_outlier_columns():
    """The tiny 64->64 layer plants columns 3 and 17 at +-U(8, 20); with threshold 6.0
    those two, and only those two, are flagged."""
    case = config_case("tiny")
    X = O.decode_bits(case.X, "f16")
    assert O.outlier_columns(X, case.threshold).tolist() == [3, 17]


def test_rows_cols_selection_matches_full():
    """Sampled evaluation equals the corresponding block of the full evaluation."""
    case = random_case(9, 50, 21, seed=11, n_out=2)
    CB, SCB = O.quantize_weight(O.decode_bits(case.W, "f16"))
    full = O.linear_forward(case.X, "f16", CB, SCB, case.bias, 6.0)
    rows, cols = [0, 4, 8], [1, 2, 20]
    part = O.linear_forward(case.X, "f16", CB, SCB, case.bias, 6.0, rows=rows, cols=cols)
    assert np.array_equal(part["idx"], full["idx"])
    assert np.array_equal(part["acc"], full["acc"][np.ix_(rows, cols)])
    assert np.array_equal(part["out_bits"], full["out_bits"][np.ix_(rows, cols)])


# ------------------------------------------------------ dtype conversions -----
def test_bf16_rounding_matches_torch():
    """The oracle's bf16 rounding agrees with torch's float32 -> bfloat16 cast
    (round to nearest even) on float32 inputs, ties included."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x00018000], np.uint32).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 1.0, 65504.0])])
    mine = O.round_to_dtype_bits(v, "bf16")
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # and decoding is the exact inverse on bf16 values
    assert np.array_equal(O.round_to_dtype_bits(O.decode_bits(mine, "bf16"), "bf16"), mine)


def test_fp16_rounding_from_float64_is_single_rounding():
    """float64 -> fp16 rounds once: 1 + 2^-11 + 2^-40 goes up although its
    float32 rounding, 1 + 2^-11, is a tie that goes to even (down)."""
    v = np.array([1 + 2.0 ** -11 + 2.0 ** -40, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], np.float64)
    bits = O.round_to_dtype_bits(v, "f16")
    assert bits.view(np.float16).astype(np.float64).tolist() == [1 + 2.0 ** -10, 1.0, 1 + 2 * 2.0 ** -10]
    vb = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8], np.float64)
    bb = O.decode_bits(O.round_to_dtype_bits(vb, "bf16"), "bf16")
    assert bb.tolist() == [1 + 2.0 ** -7, 1.0]


def test_outlier_bitmap_encoding():
    """Bit c % 32 of word c // 32 marks column c; brute-force decode gives idx back."""
    K = 100
    idx = np.array([0, 3, 31, 32, 63, 64, 99], np.int32)
    words = O.outlier_bitmap(idx, K)
    assert words.dtype == np.uint32 and words.size == 4
    back = [c for c in range(K) if (int(words[c // 32]) >> (c % 32)) & 1]
    assert back == idx.tolist()
    assert words[0] == (1 | (1 << 3) | (1 << 31))
