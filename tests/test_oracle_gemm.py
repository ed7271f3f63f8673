"""Pins for the oracle's dense product y = W x and mag = sum |W x|.

Closed forms (identity, all-equal codes, per-group scales, negation), an
exact-rational brute force on tiny shapes with the weights decoded from the
E2M1 field definition, and the row-subset entry point against the full one.
"""
from fractions import Fraction

import numpy as np
import pytest

from gemm_mxfp4_dequant_amd import inputs


def field_value(code, k):
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    v = mag * Fraction(2) ** (k - 127)
    return -v if s else v


def split_tensor(w, rows, cols):
    """Per-element codes and per-group scales read through byte pairs:
    element 2i is the low nibble of code byte i (word addressing restated)."""
    code_bytes = w[: rows * cols // 2]
    codes = np.empty(rows * cols, np.int64)
    codes[0::2] = code_bytes & 15
    codes[1::2] = code_bytes >> 4
    scales = w[rows * cols // 2: rows * cols // 2 + rows * cols // 32].astype(np.int64)
    return codes.reshape(rows, cols), scales.reshape(rows, cols // 32)


def test_identity(orc):
    n = 64
    codes = np.zeros((n, n), np.int64)
    np.fill_diagonal(codes, 2)
    flat = codes.reshape(-1)
    cb = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)
    w = np.concatenate([cb, np.full(n * n // 32, 127, np.uint8)])
    x = np.random.default_rng(1).standard_normal((3, n)).astype(np.float32)
    y, mag = orc.gemm(w, n, n, x)
    assert np.array_equal(y, x.astype(np.float64))
    assert np.array_equal(mag, np.abs(x.astype(np.float64)))


@pytest.mark.parametrize("code,value", [(2, 1.0), (10, -1.0), (7, 6.0), (9, -0.5)])
def test_all_equal_codes_sum(orc, code, value):
    rows, cols = 5, 96
    cb = np.full(rows * cols // 2, code | (code << 4), np.uint8)
    w = np.concatenate([cb, np.full(rows * cols // 32, 127, np.uint8)])
    x = np.random.default_rng(2).integers(-8, 8, size=(2, cols)).astype(np.float32)
    y, _ = orc.gemm(w, rows, cols, x)
    want = value * x.astype(np.float64).sum(axis=1)
    assert np.array_equal(y, np.repeat(want[:, None], rows, axis=1))


def test_per_group_scales_closed_form(orc):
    rows, cols = 4, 256
    rng = np.random.default_rng(3)
    scales = rng.integers(110, 140, size=(rows, cols // 32)).astype(np.uint8)
    cb = np.full(rows * cols // 2, 0x22, np.uint8)  # all code 2 (1.0)
    w = np.concatenate([cb, scales.reshape(-1)])
    x = rng.integers(-100, 100, size=(3, cols)).astype(np.float32)
    y, _ = orc.gemm(w, rows, cols, x)
    gs = x.astype(np.float64).reshape(3, cols // 32, 32).sum(axis=2)  # [b, gpr]
    want = np.einsum("bg,rg->br", gs, np.exp2(scales.astype(np.float64) - 127))
    assert np.array_equal(y, want)


def test_negated_codes_negate_output(orc):
    w, x = inputs.gemm_case(5, 8, 128, 2)
    rows, cols = 8, 128
    y, mag = orc.gemm(w, rows, cols, x)
    w2 = w.copy()
    w2[: rows * cols // 2] ^= 0x88  # flip the sign bit of both nibbles
    y2, mag2 = orc.gemm(w2, rows, cols, x)
    assert np.array_equal(y2, -y)
    assert np.array_equal(mag2, mag)


@pytest.mark.parametrize("rows,cols,b,xd", [(3, 64, 3, "f32"), (2, 96, 2, "bf16"),
                                            (4, 32, 1, "f32")])
def test_exact_rational_brute_force(orc, rows, cols, b, xd):
    """The fp64 oracle is within its summation bound of the exact rational
    product, and rounds to the same fp32 whenever the exact value is not
    within that bound of an fp32 rounding boundary."""
    w, x = inputs.gemm_case(17 + rows, rows, cols, b, 118, 132, xd)
    xf = orc._as_f64(x)
    codes, scales = split_tensor(w, rows, cols)
    y, mag = orc.gemm(w, rows, cols, x)
    u = 2.0 ** -53
    for t in range(b):
        for r in range(rows):
            exact = sum(field_value(int(codes[r, c]), int(scales[r, c // 32])) * Fraction(xf[t, c])
                        for c in range(cols))
            emag = sum(abs(field_value(int(codes[r, c]), int(scales[r, c // 32])) * Fraction(xf[t, c]))
                       for c in range(cols))
            bound = cols * u * float(emag)
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(bound), (t, r)
            assert abs(mag[t, r] - float(emag)) <= bound
            e32 = np.float32(float(exact))
            lo = np.float32(float(exact) - bound)
            hi = np.float32(float(exact) + bound)
            if lo == hi:
                assert np.float32(y[t, r]) == e32


def test_rows_subset_equals_full(orc):
    w, x = inputs.gemm_case(9, 40, 192, 3)
    y, mag = orc.gemm(w, 40, 192, x, threads=3)
    rl = np.array([0, 5, 39, 17, 17])
    ys, ms = orc.gemm_rows(w, 40, 192, x, rl, threads=2)
    assert np.array_equal(ys, y[:, rl]) and np.array_equal(ms, mag[:, rl])


def test_thread_count_does_not_change_result(orc):
    w, x = inputs.gemm_case(10, 33, 128, 2)
    y1, m1 = orc.gemm(w, 33, 128, x, threads=1)
    y4, m4 = orc.gemm(w, 33, 128, x, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(m1, m4)


def test_nan_scale_row_is_nan(orc):
    rows, cols = 3, 64
    w, x = inputs.gemm_case(12, rows, cols, 1)
    w = w.copy()
    w[rows * cols // 2 + 1 * 2 + 1] = 255  # row 1, group 1
    y, _ = orc.gemm(w, rows, cols, x)
    assert np.isnan(y[0, 1]) and np.isfinite(y[0, 0]) and np.isfinite(y[0, 2])
