"""Pins for the oracle's MXFP8 activation side (the opt-in block-scaled
FP4 x FP8 product): E4M3 decode, nearest-even encoding, the per-32-element
MX quantization, and the product with quantized activations.

* E4M3 decode: all 256 codes against the field definition (sign, exponent
  bias 7, subnormals m * 2^-9, S.1111.111 NaN, no infinities), written here
  from the definition with exact fractions;
* encoding: every finite code round-trips; each midpoint between
  neighbours goes to the even mantissa; beyond 448 saturates; below half
  the smallest subnormal flushes to zero; sign symmetry;
* quantization: hand-worked blocks (the shared exponent floor(log2 a) - 8,
  exact representation, saturation at 448, ties, zero and NaN blocks,
  elements too small for the block's scale), and a bound on the relative
  error of every element in the block's top binades;
* the product: exact-rational brute force on tiny shapes.
"""
from fractions import Fraction

import numpy as np
import pytest

from gemm_mxfp4_dequant_amd import inputs


def e4m3_field(code):
    """E4M3 value from the field definition, as a Fraction (None for NaN)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        v = Fraction(m, 2 ** 9)
    else:
        v = Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))
    return -v if s else v


def test_e4m3_all_codes(orc):
    for c in range(256):
        want = e4m3_field(c)
        got = orc.e4m3(c)
        if want is None:
            assert np.isnan(got), c
        else:
            assert Fraction(got) == want, (c, got, want)
            if c == 0x80:
                assert np.signbit(got)
    assert orc.e4m3(0x7E) == 448.0 and orc.e4m3(0x01) == 2.0 ** -9 and orc.e4m3(0x08) == 2.0 ** -6


def test_e4m3_rne(orc):
    finite = [c for c in range(0x7F)]
    vals = [float(e4m3_field(c)) for c in finite]
    for c, v in zip(finite, vals):
        assert orc.e4m3_rne(v) == c
        assert orc.e4m3_rne(-v) == (c | 0x80)
    # midpoints between neighbours: the even mantissa wins
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert orc.e4m3_rne(mid) == want, (c, mid)
        assert orc.e4m3_rne(np.nextafter(mid, 0)) == c
        assert orc.e4m3_rne(np.nextafter(mid, 1e9)) == c + 1
    # saturation and flush
    for v in (448.0, 460.0, 464.0, 479.9, 480.0, 1e6, 3e38):
        assert orc.e4m3_rne(v) == 0x7E and orc.e4m3_rne(-v) == 0xFE
    assert orc.e4m3_rne(2.0 ** -10) == 0x00          # tie with 0: even
    assert orc.e4m3_rne(2.0 ** -10 * 1.0001) == 0x01
    assert orc.e4m3_rne(-1e-30) == 0x80
    assert orc.e4m3_rne(float("nan")) == 0x7F


def quant(orc, block):
    x = np.zeros((1, 32))
    x[0, :len(block)] = block
    q, s = orc.mxfp8_quantize(x)
    return q[0], int(s[0, 0])


def test_quantize_hand_worked_blocks(orc):
    # largest 1.0: E = 0 - 8 = -8, byte 119; 1.0 / 2^-8 = 256 = 1.0 x 2^8
    q, s = quant(orc, [1.0, 0.5, -0.25, 2.0 ** -12])
    assert s == 119
    assert [orc.e4m3(c) for c in q[:4]] == [256.0, 128.0, -64.0, 2.0 ** -4]
    # 1.0625 next to 1.0: 272 lies half way between 256 and 288 -> 256 (even)
    q, s = quant(orc, [1.0, 1.0625, 1.09375])
    assert s == 119 and [orc.e4m3(c) for c in q[:3]] == [256.0, 256.0, 288.0]
    # largest 500: E = 8 - 8 = 0 (byte 127), 500 saturates to 448
    q, s = quant(orc, [500.0, -3.0])
    assert s == 127 and orc.e4m3(q[0]) == 448.0 and orc.e4m3(q[1]) == -3.0
    # largest 448 exactly: E = 0, exact
    q, s = quant(orc, [448.0, 1.0])
    assert s == 127 and orc.e4m3(q[0]) == 448.0 and orc.e4m3(q[1]) == 1.0
    # elements far below the block's largest flush to zero
    q, s = quant(orc, [1.0, 2.0 ** -19, -(2.0 ** -17)])
    assert orc.e4m3(q[1]) == 0.0 and orc.e4m3(q[2]) == -(2.0 ** -9)
    # zero block; NaN / inf blocks
    q, s = quant(orc, [])
    assert s == 0 and not q.any()
    for bad in (float("nan"), float("inf"), -float("inf")):
        q, s = quant(orc, [1.0, bad])
        assert s == 255 and not q.any()
    # scale clamps: tiny and huge blocks
    q, s = quant(orc, [2.0 ** -130])
    assert s == 0                                     # E = -138 clamps to -127
    assert orc.e4m3(q[0]) == 2.0 ** -3                # 2^-130 / 2^-127
    q, s = quant(orc, [3.0e38])                       # floor(log2 3e38) = 127
    assert s == 127 + 127 - 8 and orc.e4m3(q[0]) == 448.0   # 3e38 / 2^119 = 451.3


def test_quantize_relative_error_bound(orc):
    """Every element whose scaled magnitude lies in E4M3's normal range and
    below its largest finite value is within 2^-4 of itself; elements above
    448 under the shared scale (only the top of the block's largest binade:
    the shared exponent puts the largest in [256, 512)) saturate to 448,
    losing at most 1/8."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 256)) * np.exp2(rng.integers(-20, 20, size=(40, 1)))
    q, s = orc.mxfp8_quantize(x)
    xd = orc.mxfp8_dequantize(q, s)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    v = np.abs(x) / X
    amax = np.repeat(np.abs(x).reshape(40, 8, 32).max(axis=2), 32, axis=1)
    assert np.all((amax / X >= 256) & (amax / X < 512))
    normal = (v >= 2.0 ** -6) & (v <= 448)
    rel = np.abs(xd - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4
    sat = v > 448
    assert sat.any() and np.all(np.abs(xd[sat]) == 448 * X[sat])
    assert np.all(np.abs(xd - x)[sat] / np.abs(x)[sat] <= 1 / 8)


def test_gemm_a8_exact_brute_force(orc):
    """The product with quantized activations against exact fractions: the
    quantization redone here from the definition (shared exponent, nearest
    E4M3 by exact search) and the weights from the E2M1 field definition."""
    rows, cols, b = 3, 64, 2
    w, x = inputs.gemm_case(501, rows, cols, b, 118, 132)
    x = x.astype(np.float64)
    cb = w[: rows * cols // 2].astype(np.int64)
    codes = np.empty(rows * cols, np.int64)
    codes[0::2], codes[1::2] = cb & 15, cb >> 4
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
           Fraction(4), Fraction(6)]
    scales = w[rows * cols // 2:].astype(np.int64)
    def wv(r, c):
        n = int(codes[r * cols + c])
        v = mag[n & 7] * Fraction(2) ** (int(scales[r * (cols // 32) + c // 32]) - 127)
        return -v if n & 8 else v
    finite = [(c, e4m3_field(c)) for c in range(0x7F)]
    def nearest(v):
        a = abs(v)
        best = min(finite, key=lambda cf: (abs(a - cf[1]), cf[0] & 1))
        return -best[1] if v < 0 else best[1]
    y, _ = orc.gemm_a8(w, rows, cols, x)
    for t in range(b):
        xq = []
        for g in range(cols // 32):
            blk = [Fraction(float(v)) for v in x[t, 32 * g:32 * g + 32]]
            a = max(abs(v) for v in blk)
            E = (a.numerator.bit_length() - a.denominator.bit_length())
            if Fraction(2) ** E > a:
                E -= 1
            E -= 8
            xq += [nearest(v / Fraction(2) ** E) * Fraction(2) ** E for v in blk]
        for r in range(rows):
            exact = sum(wv(r, c) * xq[c] for c in range(cols))
            assert float(exact) == float(np.float64(y[t, r])), (t, r)
