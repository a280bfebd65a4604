"""Pins of the oracle's vector-wise quantisation variants (absmax and
zero-point, row-wise and column-wise; "Quantization mechanics": both schemes
either way).  Values the pages fix, closed forms, and invariants."""
import json
import os

import numpy as np
import pytest

import oracle.lli8_oracle as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_zeropoint_range_endpoints_and_symmetric_case():
    g = _golden("zeropoint_range_example.json")
    lo, hi = g["float_range"]
    x = np.array([[lo, -0.5, 0.0, 0.25, 0.6, hi]], np.float32)
    codes, nd, zp = M.zeropoint_quantize(x, 1)
    assert codes[0, 0] == g["code_range"][0] and codes[0, -1] == g["code_range"][1]
    assert nd[0] == np.float32(127) and zp[0] == 0
    # a range symmetric about 0: the same codes as absmax with that maximum
    ab, amax = M.absmax_quantize(x, 1)
    assert np.array_equal(codes, ab) and amax[0] == np.float32(hi)


def test_absmax_columnwise_worked_example():
    g = _golden("absmax_worked_example.json")
    col = np.array(g["vector"], np.float32)[:, None]       # one column
    codes, amax = M.absmax_quantize(col, 0)
    assert codes[:, 0].tolist() == g["codes_derived"] and amax[0] == np.float32(g["absmax"])
    rows, ramax = M.absmax_quantize(col.T, 1)
    assert np.array_equal(rows.T, codes) and ramax[0] == amax[0]


@pytest.mark.parametrize("x,nd,zp,codes", [
    ([0.0, 1.0, 2.0], 127.0, -127, [-127, 0, 127]),          # range [0, 2]
    ([-3.0, 1.0, 0.0], 63.5, 64, [-127, 127, 64]),          # 1 * 63.5 + 64 = 127.5 -> 128 -> clamped
    ([2.0, 3.0], 254.0 / 3.0, -127, [42, 127]),             # widened to [0, 3]: 2 * 84.67 - 127 = 42.3
    ([-4.0, -1.0], 63.5, 127, [-127, 63]),                  # widened to [-4, 0]: round(-63.5) = -64, + 127
])
def test_zeropoint_closed_forms(x, nd, zp, codes):
    c, n, z = M.zeropoint_quantize(np.array([x], np.float32), 1)
    assert n[0] == np.float32(254.0) / np.float32(np.float32(max(max(x), 0)) - np.float32(min(min(x), 0)))
    assert abs(float(n[0]) - nd) < 1e-4 and z[0] == zp and c[0].tolist() == codes


def test_zeropoint_all_zero_and_empty():
    c, n, z = M.zeropoint_quantize(np.zeros((3, 5), np.float32), 1)
    assert not c.any() and not n.any() and not z.any()
    c, n, z = M.zeropoint_quantize(np.zeros((2, 0), np.float32), 1)
    assert c.shape == (2, 0) and n.shape == (2,)


def _rows(seed, R=64, C=200):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((R, C)).astype(np.float32) * rng.uniform(0.01, 30, (R, 1)).astype(np.float32)
    X += rng.uniform(-5, 5, (R, 1)).astype(np.float32)      # ranges not centred on 0
    X[::7] = np.abs(X[::7])                                 # some rows all >= 0
    X[1::9] = -np.abs(X[1::9])                              # some rows all <= 0
    X[:, 3] = 0.0                                           # an exact zero in every row
    return X


@pytest.mark.parametrize("seed", [0, 1])
def test_zeropoint_invariants(seed):
    X = _rows(seed)
    codes, nd, zp = M.zeropoint_quantize(X, 1)
    assert codes.dtype == np.int8 and np.abs(codes.astype(np.int32)).max() <= 127
    assert np.all(np.abs(zp) <= 127)
    # 0.0 is exact: its code is the zero point, and it comes back as 0
    assert np.array_equal(codes[:, 3].astype(np.int32), zp)
    Xh = M.zeropoint_dequantize(codes, nd, zp, 1)
    assert np.all(Xh[:, 3] == 0.0)
    # the row's range spans the whole code range
    lo = np.minimum(X.min(axis=1), 0)
    hi = np.maximum(X.max(axis=1), 0)
    assert np.all(codes[np.arange(X.shape[0]), np.argmin(np.where(X == lo[:, None], 0, 1), axis=1)] == -127)
    # reconstruction within half a step (one step where the top end is clamped)
    step = 1.0 / nd.astype(np.float64)
    err = np.abs(Xh - X.astype(np.float64))
    assert np.all(err <= step[:, None] * (1.0 + 1e-5))
    inner = codes.astype(np.int32) < 127
    assert np.all(err[inner] <= (0.5 * step[:, None] * (1.0 + 1e-4) + 1e-6 * np.abs(X))[inner])
    # codes are monotone in x within a row
    for r in range(0, X.shape[0], 5):
        o = np.argsort(X[r], kind="stable")
        assert np.all(np.diff(codes[r, o].astype(np.int32)) >= 0)
    assert np.all(hi >= lo)


def test_zeropoint_power_of_two_scaling():
    X = _rows(3)
    c1, n1, z1 = M.zeropoint_quantize(X, 1)
    c2, n2, z2 = M.zeropoint_quantize(X * np.float32(4.0), 1)
    assert np.array_equal(c1, c2) and np.array_equal(z1, z2) and np.array_equal(n1, n2 * np.float32(4.0))


def test_columnwise_is_rowwise_of_transpose():
    X = _rows(4, R=50, C=30)
    c, n, z = M.zeropoint_quantize(X, 0)
    ct, nt, zt = M.zeropoint_quantize(np.ascontiguousarray(X.T), 1)
    assert np.array_equal(c, ct.T) and np.array_equal(n, nt) and np.array_equal(z, zt)
    a, am = M.absmax_quantize(X, 0)
    at, amt = M.absmax_quantize(np.ascontiguousarray(X.T), 1)
    assert np.array_equal(a, at.T) and np.array_equal(am, amt)


def test_zeropoint_brute_force_small():
    """Element by element with Python floats: the row's widened range, the
    step 254 / width and the code of each value, against the vectorised form."""
    rng = np.random.default_rng(9)
    X = (rng.standard_normal((6, 9)) * 3 + 1).astype(np.float32)
    codes, nd, zp = M.zeropoint_quantize(X, 1)
    for r in range(X.shape[0]):
        row = [float(v) for v in X[r]]
        lo, hi = min(min(row), 0.0), max(max(row), 0.0)
        w = float(np.float32(np.float32(hi) - np.float32(lo)))
        n = float(np.float32(254.0 / w))
        assert n == float(nd[r])
        z = int(np.floor(abs(float(np.float32(-lo * n))) + 0.5)) * (1 if -lo * n >= 0 else -1) - 127
        assert z == int(zp[r])
        for c in range(X.shape[1]):
            v = float(np.float32(row[c] * n))
            q = (1 if v >= 0 else -1) * int(np.floor(abs(v) + 0.5)) + z
            assert max(-127, min(127, q)) == int(codes[r, c])
