"""Seeded random-shape parity sweep over the C ABI (GEMM and expert bank).

Each case draws its sizes from a fixed seed so that, together, the cases
reach every launch path: the generic kernel (cols not a multiple of 512),
the split-K kernel with 512- and 1024-column slabs, one and several token
chunks, the tiled kernel (enough row blocks), fp32 and bf16 activations,
fp32 and bf16 outputs, ragged row counts; and for the expert bank the
skinny and tiled schedules with uneven routing.  Pass rules are those of
the other parity tests: |y - y_oracle| <= 1e-4 sum|w x| + 1e-30 (plus one
bf16 ulp when y is bf16); the expert bank's stage checks and end-to-end
nrmse < 1e-3, cos > 0.9999.
"""
import os

import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import assert_within, dev, host

pytestmark = pytest.mark.gpu


def gemm_cases():
    rng = np.random.default_rng(2024)
    cols_choices = [32, 96, 480, 512, 544, 1024, 1504, 2048, 3072, 4096, 5120, 8192, 12288,
                    16384]
    cases = []
    for i in range(28):
        cols = int(cols_choices[i % len(cols_choices)])
        rows = int(rng.integers(1, 2600)) if i % 7 else int(rng.integers(12300, 12600))
        if cols >= 12288:
            rows = min(rows, 700)
        b = int(rng.choice([1, 2, 3, 5, 8, 9, 16, 17, 31, 40]))
        xdt = "bf16" if rng.random() < 0.4 else "f32"
        ydt = "bf16" if rng.random() < 0.3 else "f32"
        cases.append((rows, cols, b, xdt, ydt, 5000 + i))
    # the tiled kernel with fp32 and bf16 activations, ragged last row block
    cases += [(12400, 1024, 20, "f32", "f32", 5100), (12345, 1536, 27, "f32", "bf16", 5101),
              (12300, 512, 33, "bf16", "f32", 5102)]
    return cases


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


@pytest.mark.parametrize("rows,cols,b,xdt,ydt,seed", gemm_cases())
def test_gemm_random_shapes(m, orc, rows, cols, b, xdt, ydt, seed):
    w, x = inputs.gemm_case(seed, rows, cols, b, 118, 132, xdt)
    y = m.mxfp4_gemm(dev(w), rows, cols, dev(x),
                     y_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    y = host(y)
    want, mag = orc.gemm(w, rows, cols, x)
    if ydt == "bf16":
        yf = (y.astype(np.uint32) << 16).view(np.float32)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-38))) - 7)
        assert_within(yf, want, mag, extra=ulp, what=f"{rows}x{cols} b={b} {xdt}->bf16")
    else:
        assert_within(y, want, mag, what=f"{rows}x{cols} b={b} {xdt}")


def moe_cases():
    rng = np.random.default_rng(77)
    cases = []
    for i in range(8):
        E = int(rng.integers(1, 40))
        H = int(rng.choice([64, 512, 1024, 1536]))
        I = int(rng.choice([32, 256, 512, 1024]))
        T = int(rng.integers(1, 120))
        K = int(rng.integers(1, min(E, 8) + 1))
        xdt = "bf16" if i % 2 else "f32"
        routing = "zipf" if i % 3 == 0 else "softmax"
        cases.append((E, H, I, T, K, xdt, routing, 9000 + i))
    return cases


@pytest.mark.parametrize("E,H,I,T,K,xdt,routing,seed", moe_cases())
def test_moe_random_banks(m, orc, E, H, I, T, K, xdt, routing, seed):
    from tests.test_gpu_moe import check_case
    c = inputs.moe_case(seed, E, H, I, T, K, xdt, routing, scale_lo=100, scale_hi=114)
    check_case(m, orc, c, E, H, I, xdt == "bf16")


WIDE = os.environ.get("MXFP4_WIDE_SWEEP") == "1"


@pytest.mark.skipif(not WIDE, reason="wide sweep: set MXFP4_WIDE_SWEEP=1 (about 2 minutes per seed)")
@pytest.mark.parametrize("seed", [11, 23])
def test_wide_random_sweep(m, orc, seed):
    """150 random GEMMs (up to 70000 rows, so that workgroups walk several
    row blocks; fp32/bf16 in and out; 1-64 tokens) and 40 random expert
    banks (up to 130 experts, decode-sized banks with 4096 hidden columns
    among them); every failure is collected before the assert."""
    from tests.test_gpu_moe import check_case
    rng = np.random.default_rng(seed)
    fails = []
    cols_choices = [32, 64, 96, 480, 512, 544, 1024, 1504, 2048, 2080, 3072, 4096, 5120, 7168,
                    8192, 16384]
    for i in range(150):
        cols = int(rng.choice(cols_choices))
        r = rng.random()
        if r < 0.15:
            rows, cols = int(rng.integers(33000, 70000)), min(cols, 1024)
        elif r < 0.35:
            rows, cols = int(rng.integers(10000, 15000)), min(cols, 4096)
        else:
            rows = int(rng.integers(1, 5000))
        if cols >= 8192:
            rows = min(rows, 1500)
        b = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 23, 24, 31, 32, 33, 40, 48, 64]))
        xdt = "bf16" if rng.random() < 0.4 else "f32"
        ydt = "bf16" if rng.random() < 0.25 else "f32"
        try:
            test_gemm_random_shapes(m, orc, rows, cols, b, xdt, ydt, 70000 + i)
        except AssertionError as e:
            fails.append(("gemm", rows, cols, b, xdt, ydt, str(e)[:200]))
    for i in range(40):
        if i % 5 == 0:
            E, H = int(rng.choice([32, 64])), 4096
            I, T, K = int(rng.choice([2048, 2080, 1024])), int(rng.integers(4, 12)), int(
                rng.integers(4, 9))
        else:
            E = int(rng.integers(1, 130))
            H = int(rng.choice([64, 512, 1024, 1536, 2048, 4096]))
            I = int(rng.choice([32, 256, 512, 1024, 2048]))
            T = int(rng.integers(1, 200))
            K = int(rng.integers(1, min(E, 8) + 1))
            if H * I > 2048 * 2048 and E > 32:
                E = 32
        xdt = "bf16" if rng.random() < 0.5 else "f32"
        routing = "zipf" if rng.random() < 0.3 else "softmax"
        c = inputs.moe_case(80000 + i, E, H, I, T, K, xdt, routing, scale_lo=100, scale_hi=114)
        try:
            check_case(m, orc, c, E, H, I, xdt == "bf16")
        except AssertionError as e:
            fails.append(("moe", E, H, I, T, K, xdt, routing, str(e)[:200]))
    assert not fails, fails
