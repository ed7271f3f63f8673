"""Pins for the oracle's reading of the stored layout.

The placement rules are checked against an independent restatement of the
pages' addressing ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", PEROP
shader): a tensor is an array of little-endian u32 words; row r, group g
occupies words (r*gpr + g)*4 .. +4, and nibble j of word q is column
32g + 8q + j; the scale bytes follow the code words at byte r*gpr + g of the
scale plane (mx_scale).  Fixtures are built word by word here, never with
the oracle's own byte/nibble formula.
"""
import json
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")))


def build_words(rows, cols, code_fn, scale_fn):
    """Stored bytes from per-element codes and per-group scales, assembled
    through the shader's word addressing."""
    gpr = cols // 32
    words = np.zeros(rows * gpr * 4, np.uint32)
    for r in range(rows):
        for g in range(gpr):
            for q in range(4):
                word = 0
                for j in range(8):
                    word |= (code_fn(r, 32 * g + 8 * q + j) & 15) << (4 * j)
                words[(r * gpr + g) * 4 + q] = word
    scales = np.array([scale_fn(r, g) for r in range(rows) for g in range(gpr)], np.uint8)
    return np.concatenate([words.astype("<u4").view(np.uint8), scales])


def test_codec_lengths_match_pages(orc):
    cl = GOLD["codec_lengths"]
    assert orc.nbytes(2304, 5120) == cl["2304x5120"] == 2304 * 5120 * 17 // 32
    assert orc.nbytes(5120, 2304) == cl["5120x2304"]
    assert orc.nbytes(1, 32) == cl["1x32"] == 17
    assert orc.nbytes(4, 48) == -1  # cols not a multiple of 32


@pytest.mark.parametrize("rows,cols", [(3, 64), (5, 96), (2, 256)])
def test_one_hot_code_lights_one_weight(orc, rows, cols):
    """A single code 2 (value 1.0, scale byte 127) at (r, c) dequantizes to a
    matrix whose only nonzero is 1.0 at (r, c), and the product with x picks
    x[c] for row r only."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, cols)).astype(np.float32)
    picks = [(0, 0), (rows - 1, cols - 1), (rows // 2, 31), (rows // 2, 32), (1, 8), (1, 7)]
    for (r0, c0) in picks:
        w = build_words(rows, cols, lambda r, c: 2 if (r, c) == (r0, c0) else 0,
                        lambda r, g: 127)
        d = orc.dequant_f32(w, rows, cols)
        want = np.zeros((rows, cols), np.float32)
        want[r0, c0] = 1.0
        assert np.array_equal(d, want)
        y, mag = orc.gemm(w, rows, cols, x)
        exp = np.zeros((2, rows))
        exp[:, r0] = x[:, c0]
        assert np.array_equal(y, exp)
        assert np.array_equal(mag, np.abs(exp))


def test_one_hot_scale_reaches_one_group(orc):
    """All codes 2; one group's scale byte raised: exactly that (row, group)
    block changes, by the factor 2^(k-127)."""
    rows, cols = 4, 128
    gpr = cols // 32
    for (r0, g0) in [(0, 0), (3, 3), (2, 1)]:
        w = build_words(rows, cols, lambda r, c: 2,
                        lambda r, g: 130 if (r, g) == (r0, g0) else 127)
        d = orc.dequant_f32(w, rows, cols)
        want = np.ones((rows, cols), np.float32)
        want[r0, 32 * g0:32 * g0 + 32] = 8.0
        assert np.array_equal(d, want)
    assert gpr == 4


def test_random_tensor_matches_word_assembly(orc):
    """A random tensor assembled word by word decodes to the exact values of
    its per-element codes and per-group scales."""
    rng = np.random.default_rng(11)
    rows, cols = 6, 160
    codes = rng.integers(0, 16, size=(rows, cols))
    scales = rng.integers(100, 150, size=(rows, cols // 32))
    w = build_words(rows, cols, lambda r, c: int(codes[r, c]), lambda r, g: int(scales[r, g]))
    d = orc.dequant_f32(w, rows, cols)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    want = np.where(codes >= 8, -1.0, 1.0) * mags[codes & 7] * np.exp2(
        np.repeat(scales, 32, axis=1) - 127.0)
    assert np.array_equal(d.astype(np.float64), want)
    assert np.array_equal(np.signbit(d), codes >= 8)
