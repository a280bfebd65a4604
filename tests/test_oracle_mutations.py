"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Every case patches one step of the oracle module, reruns the pin test that
guards that step, and expects it to fail.  This shows the pins are not
vacuous: a dropped term, a wrong comparison, rounding mode, scale, axis,
order or sign, or a transposed operand all break at least one of them.
"""
import numpy as np
import pytest

import oracle.lli8_oracle as M
import tests.test_oracle_pins as P


def _rint(v):
    return np.rint(np.asarray(v, np.float64))


def _outliers_ge(X, threshold):
    tau = np.float32(threshold)
    if not tau > 0:
        return np.zeros(0, np.int32)
    return np.nonzero(np.max(np.abs(X), axis=0) >= tau)[0].astype(np.int32)


def _absmax_no_exclusion(X, excluded_cols=None):
    return _orig_absmax(X, None)


def _dequant_127(acc, SCA, SCB):
    return acc.astype(np.float64) * SCA[:, None] * SCB[None, :] / 127.0


def _recover_no_div(CB_cols, SCB, dtype):
    prod = CB_cols.astype(np.float32) * SCB.astype(np.float32)[:, None]
    return M.decode_bits(M.round_to_dtype_bits(prod, dtype), dtype).astype(np.float64)


def _acc_transposed_weight(CA, CB, chunk=4096):
    # uses CB's columns in reverse order, a plausible indexing slip
    return _orig_acc(CA, CB[:, ::-1].copy(), chunk)


def _scale_div_not_mul(X, excluded_cols=None):
    codes, amax = _orig_absmax(X, excluded_cols)
    # codes from x / 127 * absmax-style slip: wrong scale direction
    live = amax > 0
    Xr = np.array(X, np.float32, copy=True)
    if excluded_cols is not None and len(excluded_cols):
        Xr[:, np.asarray(excluded_cols)] = 0
    v = Xr[live] * (amax[live] / np.float32(127))[:, None]
    codes = codes.copy()
    codes[live] = np.clip(M.round_half_away(v), -127, 127).astype(np.int8)
    return codes, amax


def _outliers_over_rows(X, threshold):
    # the maximum taken along the wrong axis: flags rows, not feature columns
    tau = np.float32(threshold)
    if not tau > 0 or X.shape[0] == 0:
        return np.zeros(0, np.int32)
    return np.nonzero(np.max(np.abs(X), axis=1) > tau)[0].astype(np.int32)


def _outliers_descending(X, threshold):
    return _orig_outliers(X, threshold)[::-1].copy()


def _outliers_signed(X, threshold):
    # x > tau instead of |x| > tau: large negative values are missed
    tau = np.float32(threshold)
    if not tau > 0 or X.shape[0] == 0:
        return np.zeros(0, np.int32)
    return np.nonzero(np.max(X, axis=0) > tau)[0].astype(np.int32)


def _weight_scale_per_input_feature(W):
    # one scale per column of W [N, K] instead of per output row
    codes, amax = _orig_absmax(np.asarray(W, np.float32).T, None)
    return codes.T.copy(), amax


def _signed_row_max(X, excluded_cols=None):
    # max(x) instead of max(|x|): rows led by a negative value get clipped codes
    X = np.array(X, np.float32, copy=True)
    if excluded_cols is not None and len(excluded_cols):
        X[:, np.asarray(excluded_cols)] = 0
    amax = (np.max(X, axis=1) if X.shape[1] else np.zeros(X.shape[0], np.float32)).astype(np.float32)
    amax = np.maximum(amax, np.float32(0))
    codes = np.zeros(X.shape, np.int8)
    live = amax > 0
    if np.any(live):
        v = X[live] * (np.float32(127) / amax[live])[:, None]
        codes[live] = np.clip(M.round_half_away(v), -127, 127).astype(np.int8)
    return codes, amax


_orig_absmax = M.absmax_quantize_rows
_orig_acc = M.int8_accumulate
_orig_outliers = M.outlier_columns


def _reload_pins(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    # the pin module calls through the package namespace; patch it there too
    import oracle
    monkeypatch.setattr(oracle, name, fn)


MUTATIONS = [
    ("round_half_away", _rint, P.test_rounding_is_half_away_from_zero, ()),
    ("outlier_columns", _outliers_ge, P.test_threshold_is_strict, ()),
    ("absmax_quantize_rows", _absmax_no_exclusion,
     P.test_output_within_apriori_error_bound, ("f16", 0)),
    ("dequantize", _dequant_127, P.test_output_within_apriori_error_bound, ("f16", 1)),
    ("recover_weight", _recover_no_div, P.test_weight_recovery_bound, ("f16",)),
    ("int8_accumulate", _acc_transposed_weight, P.test_integer_special_case_is_textbook_matmul, ()),
    ("absmax_quantize_rows", _scale_div_not_mul, P.test_absmax_worked_example_fp32, ()),
    ("outlier_columns", _outliers_over_rows, P.test_issue_tiny_threshold_flags_every_column, ()),
    ("outlier_columns", _outliers_descending, P.test_tiny_config_outlier_columns, ()),
    ("outlier_columns", _outliers_signed, P.test_threshold_is_strict, ()),
    ("quantize_weight", _weight_scale_per_input_feature, P.test_weight_bits_worked_example_and_row_selection, ()),
    ("absmax_quantize_rows", _signed_row_max, P.test_weight_bits_worked_example_and_row_selection, ()),
]


@pytest.mark.parametrize("name,fn,pin,args", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pin, args):
    _reload_pins(monkeypatch, name, fn)
    with pytest.raises(AssertionError):
        pin(*args)


def test_dropped_outlier_term_is_caught(monkeypatch):
    """Drop the 16-bit outlier product: the a priori bound test fails."""
    orig = M.linear_forward

    def no_outlier_forward(X_bits, dtype, CB, SCB, bias_bits, threshold, rows=None, cols=None):
        r = orig(X_bits, dtype, CB, SCB, bias_bits, threshold, rows, cols)
        X = M.decode_bits(X_bits, dtype)
        if r["idx"].size:
            What = M.recover_weight(CB[:, r["idx"]], SCB, dtype)
            r["out64"] = r["out64"] - X[:, r["idx"]].astype(np.float64) @ What.T
        return r

    _reload_pins(monkeypatch, "linear_forward", no_outlier_forward)
    with pytest.raises(AssertionError):
        P.test_output_within_apriori_error_bound("bf16", 2)


def test_dropped_bias_is_caught(monkeypatch):
    """Drop the bias from the output sum: the a priori bound test fails."""
    orig = M.linear_forward

    def no_bias_forward(X_bits, dtype, CB, SCB, bias_bits, threshold, rows=None, cols=None):
        return orig(X_bits, dtype, CB, SCB, None, threshold, rows, cols)

    _reload_pins(monkeypatch, "linear_forward", no_bias_forward)
    with pytest.raises(AssertionError):
        P.test_output_within_apriori_error_bound("f16", 3)
