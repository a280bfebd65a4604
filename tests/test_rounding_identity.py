"""Why the GPU quantisers may round with one conversion.

The codes are round_half_away(v) for v = fl32(|x| * s), 0 <= v <= 127.5, with
s = fl32(127 / absmax).  For v >= 0 that is floor(v + 0.5), which
v_cvt_rpi_i32_f32 computes.  If the hardware rounded v + 0.5 to float32 before
the floor, the result would change at exactly one value: v = 0.5 - 2^-25, where
fl32(v + 0.5) = 1.0 (below 0.25 the sum stays under 0.75; from 0.5 upward 0.5
is a multiple of the spacing, so the sum is exact).  These tests pin both
facts, and show that no fp16 or bf16 input can produce that value, so the codes
are the same either way.

They also keep the alternative the kernels used before: with mantissa bit 0 of
v cleared first, fl32(v' + 0.5) is exact for every v in range.  The
zero-point codes use that form, for |v| <= 254 (their scale is 254 / range,
for which the trap is not ruled out): the last two tests pin it there.
"""
import numpy as np

TRAP = np.float32(0.5) - np.float32(2.0 ** -25)


def test_half_away_identity_exhaustive():
    """floor(fl32(v' + 0.5)) == floor(v + 0.5) for every float32 in [0, 127.5]."""
    hi = int(np.float32(127.5).view(np.uint32))
    step = 1 << 25
    for s in range(0, hi + 1, step):
        b = np.arange(s, min(s + step, hi + 1), dtype=np.uint32)
        v = b.view(np.float32)
        ref = np.floor(v.astype(np.float64) + 0.5)
        w = (b & np.uint32(0xFFFFFFFE)).view(np.float32) + np.float32(0.5)
        assert np.array_equal(np.trunc(w).astype(np.float64), ref), hex(s)


def test_rounded_sum_differs_only_at_the_trap():
    """fl32(v + 0.5) changes floor(v + 0.5) for exactly one float32 in [0, 127.5]."""
    hi = int(np.float32(127.5).view(np.uint32))
    step = 1 << 25
    bad = []
    for s in range(0, hi + 1, step):
        b = np.arange(s, min(s + step, hi + 1), dtype=np.uint32)
        v = b.view(np.float32)
        ref = np.floor(v.astype(np.float64) + 0.5)
        got = np.floor((v + np.float32(0.5)).astype(np.float64))
        bad.extend(b[got != ref].tolist())
    assert bad == [int(TRAP.view(np.uint32))]


def _trap_products(ms, xs_of_m, s):
    """(m, x) pairs with fl32(x * s) == TRAP, x among a few values near TRAP / s."""
    hits = []
    for cand in xs_of_m:
        v = (cand * s).astype(np.float32)
        ok = (v.view(np.uint32) == TRAP.view(np.uint32)) & (cand <= ms)
        hits += list(zip(ms[ok].tolist(), cand[ok].tolist()))
    return hits


def test_no_fp16_input_reaches_the_trap():
    """For every fp16 absmax m and fp16 x <= m, fl32(x * fl32(127 / m)) != 0.5 - 2^-25.
    v is increasing in x, so only the few fp16 values next to TRAP / s can hit it."""
    ms = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    s = (np.float32(127) / ms).astype(np.float32)
    target = (TRAP.astype(np.float64) / s.astype(np.float64)).astype(np.float16).view(np.uint16).astype(np.int32)
    cands = [np.clip(target + d, 1, 0x7BFF).astype(np.uint16).view(np.float16).astype(np.float32)
             for d in range(-3, 4)]
    assert _trap_products(ms, cands, s) == []


def test_no_bf16_input_reaches_the_trap():
    """The same for bf16 absmax values whose scale 127 / m is finite."""
    mb = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    ms = (mb << np.uint32(16)).view(np.float32)
    with np.errstate(over="ignore", divide="ignore"):
        s = (np.float32(127) / ms).astype(np.float32)
    keep = np.isfinite(s)
    ms, s = ms[keep], s[keep]
    t = (TRAP.astype(np.float64) / s.astype(np.float64)).astype(np.float32).view(np.uint32) >> np.uint32(16)
    cands = [((np.clip(t.astype(np.int64) + d, 1, 0x7F7F).astype(np.uint32)) << np.uint32(16)).view(np.float32)
             for d in range(-3, 4)]
    assert _trap_products(ms, cands, s) == []


def test_plain_add_half_has_the_trap():
    assert np.trunc(TRAP + np.float32(0.5)) == 1.0   # the rounded sum reaches 1 at the trap


def test_cleared_bit_zero_keeps_every_tie():
    """With mantissa bit 0 cleared, v' = v or v less one ulp; floor(v' + 0.5)
    differs from floor(v + 0.5) only if v is a tie k + 0.5 with that bit set.
    No tie below 256 has it set, so the exact-sum form is unchanged too."""
    ties = (np.arange(256, dtype=np.float64) + 0.5).astype(np.float32)
    assert np.array_equal((ties.astype(np.float64) - np.arange(256)), np.full(256, 0.5))  # exact ties
    assert not np.any(ties.view(np.uint32) & np.uint32(1))


def test_half_away_identity_zero_point_range():
    """floor(fl32(v' + 0.5)) == floor(v + 0.5) for every float32 in [127.5, 256]
    (v' = v with mantissa bit 0 cleared; [0, 127.5] is the first test)."""
    lo = int(np.float32(127.5).view(np.uint32))
    hi = int(np.float32(256.0).view(np.uint32))
    b = np.arange(lo, hi + 1, dtype=np.uint32)
    v = b.view(np.float32)
    ref = np.floor(v.astype(np.float64) + 0.5)
    w = (b & np.uint32(0xFFFFFFFE)).view(np.float32) + np.float32(0.5)
    assert np.array_equal(np.trunc(w).astype(np.float64), ref)
