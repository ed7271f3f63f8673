"""Pins for the oracle's bf16 rounding (used for the MoE outputs).

Checked against (1) an exact rational nearest-even search over the bf16
grid, and (2) for fp32 inputs, the pages' rounding rule from the GLOBAL
shader of "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" (mxg_bf16:
bits + 0x7FFF + ((bits >> 16) & 1), then clear the low half; inf and NaN
pass through), which is the same nearest-even rule applied to fp32.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest


def bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def exact_nearest_even(v):
    """Nearest bf16 to v (a finite float) by exact search; ties to the even
    significand; overflow to inf past max + half an ulp."""
    fv = Fraction(v)
    a = abs(fv)
    sign = 0x8000 if (v < 0 or (v == 0 and math.copysign(1, v) < 0)) else 0
    if a == 0:
        return sign
    maxf = Fraction(bf16_value(0x7F7F))
    if a >= maxf + Fraction(2) ** (127 - 8):  # half an ulp above the largest
        return sign | 0x7F80
    # candidates: the two neighbours among non-negative bf16 values
    lo_bits = 0
    hi_bits = 0x7F7F
    while hi_bits - lo_bits > 1:   # binary search on the monotone bit pattern
        mid = (lo_bits + hi_bits) // 2
        if Fraction(bf16_value(mid)) <= a:
            lo_bits = mid
        else:
            hi_bits = mid
    if Fraction(bf16_value(hi_bits)) <= a:
        lo_bits = hi_bits
        hi_bits = hi_bits + 1
    dl = a - Fraction(bf16_value(lo_bits))
    dh = Fraction(bf16_value(hi_bits)) - a if hi_bits <= 0x7F7F else None
    if dh is None or dl < dh:
        pick = lo_bits
    elif dh < dl:
        pick = hi_bits
    else:
        pick = lo_bits if lo_bits % 2 == 0 else hi_bits
    return sign | pick


def pages_rule(f32):
    bits = struct.unpack("<I", struct.pack("<f", f32))[0]
    if (bits & 0x7F800000) == 0x7F800000:
        return bits >> 16
    r = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFFFFFF
    return (r & 0xFFFF0000) >> 16


def test_random_fp64_values(orc):
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 130, 400)))
    vals += [1.0, -1.0, 0.0, -0.0, 3.0e38, -3.4e38, 1e-40, -1e-45, 2.0 ** -133, 2.0 ** -134]
    for v in vals:
        assert orc.bf16_rne(v) == exact_nearest_even(float(v)), v


def test_ties_go_to_even(orc):
    one = Fraction(1)
    ulp = Fraction(1, 128)
    for k in range(20):
        mid = one + (2 * k + 1) * ulp / 2  # halfway between two bf16 values
        v = float(mid)
        got = orc.bf16_rne(v)
        assert got == exact_nearest_even(v)
        assert got % 2 == 0
    # just above and just below a tie
    v = 1.0 + 2 ** -8
    assert orc.bf16_rne(v) == 0x3F80
    assert orc.bf16_rne(math.nextafter(v, 2)) == 0x3F81


def test_special_values(orc):
    assert orc.bf16_rne(float("nan")) == 0x7FC0
    assert orc.bf16_rne(float("inf")) == 0x7F80
    assert orc.bf16_rne(float("-inf")) == 0xFF80
    assert orc.bf16_rne(-0.0) == 0x8000
    big = bf16_value(0x7F7F)
    assert orc.bf16_rne(big) == 0x7F7F
    assert orc.bf16_rne(float(Fraction(big) + Fraction(2) ** 119)) == 0x7F80  # tie -> even = inf


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_pages_rule_on_fp32(orc, seed):
    rng = np.random.default_rng(seed)
    f = (rng.standard_normal(2000) * np.exp2(rng.integers(-120, 120, 2000))).astype(np.float32)
    raw = rng.integers(0, 2 ** 32, 500, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f = np.concatenate([f, raw[np.isfinite(raw)]])
    for v in f:
        assert orc.bf16_rne(float(v)) == pages_rule(float(v)), float(v)
