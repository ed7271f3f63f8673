"""Pins for the oracle's format decode (E2M1, E8M0, per-weight dequant).

Each check compares the oracle with something other than itself:
  * the OCP E2M1 field definition (sign bit, 2-bit exponent with bias 1,
    1-bit mantissa, subnormal when the exponent field is 0), decoded here as
    exact rationals;
  * the pages' own bit construction from the DECODE shader of
    "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" (mx_e2m1: 0x3F000000 +
    m<<22 with 0 and 0.5 patched; mx_e8m0: k<<23, 0x00400000, 0x7FC00000);
  * the golden table in tests/golden/mxfp4_format.json (same page, cited).
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")))


def f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bits_of_f32(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def e2m1_fields(n):
    """OCP E2M1: s | e1 e0 | m, bias 1; e == 0 is subnormal (m * 1/2)."""
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = n & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return s, mag


def shader_e2m1(n):
    """The pages' mx_e2m1 construction, evaluated in fp32."""
    m = n & 7
    v = np.float32(f32_from_bits(0x3F000000 + (m << 22)))
    if m == 0:
        v = np.float32(0.0)
    if m == 1:
        v = np.float32(0.5)
    return -v if (n & 8) else v


def shader_e8m0(k):
    if k == 255:
        return np.float32(f32_from_bits(0x7FC00000))
    if k == 0:
        return np.float32(f32_from_bits(0x00400000))
    return np.float32(f32_from_bits(k << 23))


@pytest.mark.parametrize("n", range(16))
def test_e2m1_matches_field_definition(orc, n):
    s, mag = e2m1_fields(n)
    v = orc.e2m1(n)
    assert Fraction(abs(v)) == mag
    assert math.copysign(1.0, v) == (-1.0 if s else 1.0)  # includes -0 for code 8


def test_e2m1_matches_shader_and_golden(orc):
    for n in range(16):
        ov = np.float32(orc.e2m1(n))
        sv = shader_e2m1(n)
        assert bits_of_f32(ov) == bits_of_f32(sv), n
        assert "0x%08X" % bits_of_f32(ov) == GOLD["e2m1_f32_bits"][n]
        assert math.copysign(1, GOLD["e2m1_codes_0_to_15"][n]) == math.copysign(1, ov)


def test_e8m0_all_256(orc):
    for k in range(256):
        ov = orc.e8m0(k)
        sv = shader_e8m0(k)
        if k == 255:
            assert math.isnan(ov) and math.isnan(sv)
            continue
        assert ov == Fraction(2) ** (k - 127)  # exact value 2^(k-127)
        assert ov == float(sv), k             # and the shader's bit pattern
    assert GOLD["e8m0_f32_bits"]["0"] == "0x%08X" % bits_of_f32(np.float32(orc.e8m0(0)))


def test_dequant_all_4096_pairs_bitwise(orc):
    """Every (code, scale) pair: the oracle's fp32 weight equals the exact
    rational product rounded once to fp32 (with +-inf on overflow), and equals
    the fp32 product of the shader's two decodes (an exact IEEE product or its
    overflow).  NaN scale gives the canonical 0x7FC00000 (the build's reading)."""
    with np.errstate(over="ignore"):
        for k in range(256):
            for n in range(16):
                got = orc.dequant_value_f32(n, k)
                gb = bits_of_f32(got)
                if k == 255:
                    assert gb == 0x7FC00000
                    continue
                s, mag = e2m1_fields(n)
                exact = mag * Fraction(2) ** (k - 127)
                if exact >= Fraction(2) ** 128:
                    want = np.float32(np.inf)
                else:
                    want = np.float32(float(exact))
                    assert Fraction(float(want)) == exact  # exactly representable
                if s:
                    want = -want
                assert gb == bits_of_f32(want), (n, k)
                prod = np.float32(shader_e2m1(n) * shader_e8m0(k))
                assert gb == bits_of_f32(prod), (n, k)


def test_dequant_covers_edge_classes(orc):
    """The exhaustive set above includes -0, subnormal, overflow and NaN."""
    assert bits_of_f32(orc.dequant_value_f32(8, 127)) == 0x80000000          # -0
    assert bits_of_f32(orc.dequant_value_f32(1, 0)) == 0x00200000            # 2^-128
    assert bits_of_f32(orc.dequant_value_f32(3, 0)) == 0x00600000            # 1.5*2^-127
    assert np.isinf(orc.dequant_value_f32(4, 254))                           # 2*2^127
    assert np.isfinite(orc.dequant_value_f32(3, 254))                        # 1.5*2^127
    assert np.isinf(orc.dequant_value_f32(14, 253)) and orc.dequant_value_f32(14, 253) < 0
    assert np.isfinite(orc.dequant_value_f32(5, 253))                        # 3*2^126


def test_dequant_bf16_is_top_half_of_exact_f32(orc):
    """All 4096 pairs as a 1 x 4096 tensor... built as 128 rows x 32 columns:
    row r carries scale r (for r < 128) and then 128..255 in a second tensor."""
    for base in (0, 128):
        rows, cols = 128, 32
        codes = np.zeros(rows * cols // 2, np.uint8)
        nib = np.tile(np.arange(16, dtype=np.uint8), rows * cols // 16)
        codes[:] = nib[0::2] | (nib[1::2] << 4)
        scales = np.arange(base, base + rows, dtype=np.uint8)
        w = np.concatenate([codes, scales])
        f = orc.dequant_f32(w, rows, cols)
        h = orc.dequant_bf16(w, rows, cols)
        fb = f.view(np.uint32)
        finite = np.isfinite(f)
        assert np.all((fb[finite] & 0xFFFF) == 0)
        assert np.array_equal(h[finite], (fb[finite] >> 16).astype(np.uint16))
        nan = np.isnan(f)
        assert np.all(h[nan] == 0x7FC0)
        inf = np.isinf(f)
        assert np.array_equal(h[inf], (fb[inf] >> 16).astype(np.uint16))
