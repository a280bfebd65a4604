"""The GPU quantisers round half away from zero with a short sequence:
for 0 <= v <= 127.5 (every |x| * s the codes can see),

    round_half_away(v) == trunc(fl32(v' + 0.5)),  v' = v with mantissa bit 0 cleared.

Clearing bit 0 makes v' + 0.5 exact in float32 (it can only move into the next
binade, whose spacing is twice v's), and never moves v across a half-integer
(half-integers below 2^22 have bit 0 clear).  The plain fl32(v + 0.5) fails at
v = 0.5 - 2^-25.  This checks the identity for every float32 in [0, 127.5]
(numpy float32 addition rounds to nearest even, as the GPU's v_add_f32 does).
"""
import numpy as np


def test_half_away_identity_exhaustive():
    hi = int(np.float32(127.5).view(np.uint32))
    step = 1 << 25
    for s in range(0, hi + 1, step):
        b = np.arange(s, min(s + step, hi + 1), dtype=np.uint32)
        v = b.view(np.float32)
        ref = np.floor(v.astype(np.float64) + 0.5)
        w = (b & np.uint32(0xFFFFFFFE)).view(np.float32) + np.float32(0.5)
        assert np.array_equal(np.trunc(w).astype(np.float64), ref), hex(s)


def test_plain_add_half_has_the_trap():
    v = np.nextafter(np.float32(0.5), np.float32(0))
    assert np.trunc(v + np.float32(0.5)) == 1.0   # the naive form rounds 0.49999997 up
