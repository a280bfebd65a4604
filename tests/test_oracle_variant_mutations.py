"""Plant plausible mistakes in the oracle's zero-point quantiser (on the CPU)
and check that one of its pins fails for each: a 255-wide scale, a zero point
without the -127 shift, a range not widened to contain 0, half-to-even
rounding, the zero point added before the rounding, the zero point taken from
the top of the range."""
import numpy as np
import pytest

import oracle.lli8_oracle as M
import tests.test_oracle_variants as P

_orig = M.zeropoint_quantize_rows


def _variant(scale=254.0, shift=127, widen=True, rnd=None):
    rnd = rnd or M.round_half_away

    def q(X):
        X = np.asarray(X, dtype=np.float32)
        R, C = X.shape
        if C == 0:
            return np.zeros((R, 0), np.int8), np.zeros(R, np.float32), np.zeros(R, np.int32)
        lo, hi = X.min(axis=1), X.max(axis=1)
        if widen:
            lo, hi = np.minimum(lo, np.float32(0)), np.maximum(hi, np.float32(0))
        width = (hi - lo).astype(np.float32)
        nd = np.zeros(R, np.float32)
        zp = np.zeros(R, np.int32)
        codes = np.zeros((R, C), np.int8)
        live = width > 0
        nd[live] = np.float32(scale) / width[live]
        zp[live] = (rnd((-lo[live] * nd[live]).astype(np.float32)) - shift).astype(np.int32)
        v = X[live] * nd[live][:, None]
        codes[live] = np.clip(rnd(v) + zp[live][:, None], -127, 127).astype(np.int8)
        return codes, nd, zp
    return q


def _half_even(v):
    return np.rint(np.asarray(v, np.float64))


def _shifted_rounding(zp_from_top):
    """The two remaining slips in the code and zero-point formulas: the zero
    point added before the rounding (round(x * nd + zp)), or the zero point
    taken from the top of the range (127 - round(hi * nd))."""
    def q(X):
        X = np.asarray(X, dtype=np.float32)
        R, C = X.shape
        if C == 0:
            return np.zeros((R, 0), np.int8), np.zeros(R, np.float32), np.zeros(R, np.int32)
        lo = np.minimum(X.min(axis=1), np.float32(0)).astype(np.float32)
        hi = np.maximum(X.max(axis=1), np.float32(0)).astype(np.float32)
        width = (hi - lo).astype(np.float32)
        nd = np.zeros(R, np.float32)
        zp = np.zeros(R, np.int32)
        codes = np.zeros((R, C), np.int8)
        live = width > 0
        nd[live] = np.float32(254.0) / width[live]
        v = (X[live] * nd[live][:, None]).astype(np.float32)
        if zp_from_top:
            zp[live] = (127 - M.round_half_away((hi[live] * nd[live]).astype(np.float32))).astype(np.int32)
            q8 = M.round_half_away(v) + zp[live][:, None]
        else:
            zp[live] = (M.round_half_away((-lo[live] * nd[live]).astype(np.float32)) - 127).astype(np.int32)
            q8 = M.round_half_away(v + zp[live][:, None].astype(np.float32))
        codes[live] = np.clip(q8, -127, 127).astype(np.int8)
        return codes, nd, zp
    return q


PINS = [P.test_zeropoint_range_endpoints_and_symmetric_case,
        lambda: [P.test_zeropoint_closed_forms(*c) for c in (
            ([0.0, 1.0, 2.0], 127.0, -127, [-127, 0, 127]),
            ([-3.0, 1.0, 0.0], 63.5, 64, [-127, 127, 64]),
            ([2.0, 3.0], 254.0 / 3.0, -127, [42, 127]),
            ([-4.0, -1.0], 63.5, 127, [-127, 63]))],
        lambda: P.test_zeropoint_invariants(0),
        P.test_zeropoint_brute_force_small]


@pytest.mark.parametrize("mutant", [
    _variant(scale=255.0), _variant(shift=0), _variant(widen=False), _variant(rnd=_half_even),
    _shifted_rounding(False), _shifted_rounding(True)],
    ids=["scale-255", "no-shift", "range-not-widened", "half-even", "zp-before-rounding", "zp-from-top"])
def test_a_pin_catches(mutant, monkeypatch):
    monkeypatch.setattr(M, "zeropoint_quantize_rows", mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_unmutated_passes_every_pin():
    for pin in PINS:
        pin()
