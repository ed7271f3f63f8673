"""GPU parity: mxfp4_dequant is bit-exact against the oracle (fp32 and bf16),
on all 4096 (code, scale) pairs including -0, subnormal, overflow and NaN,
on ragged random tensors, and on a full 14336 x 4096 tensor."""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def all_pairs_tensor(base):
    rows, cols = 128, 32
    nib = np.tile(np.arange(16, dtype=np.uint8), rows * cols // 16)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    scales = np.arange(base, base + rows, dtype=np.uint8)
    return np.concatenate([codes, scales]), rows, cols


@pytest.mark.parametrize("base", [0, 128])
def test_all_pairs_bitwise(m, orc, base):
    w, rows, cols = all_pairs_tensor(base)
    wd = dev(w)
    f = host(m.mxfp4_dequant(wd, rows, cols, out_dtype=torch.float32))
    b = host(m.mxfp4_dequant(wd, rows, cols, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(f.view(np.uint32), orc.dequant_f32(w, rows, cols).view(np.uint32))
    assert np.array_equal(b, orc.dequant_bf16(w, rows, cols))


@pytest.mark.parametrize("rows,cols,lo,hi", [(1, 32, 0, 255), (3, 96, 0, 255), (37, 160, 100, 150),
                                            (300, 2304, 118, 132), (5, 5120, 0, 255)])
def test_random_bitwise(m, orc, rows, cols, lo, hi):
    w, _ = inputs.gemm_case(rows * 7 + cols, rows, cols, 1, lo, hi)
    wd = dev(w)
    f = host(m.mxfp4_dequant(wd, rows, cols, out_dtype=torch.float32))
    b = host(m.mxfp4_dequant(wd, rows, cols, out_dtype=torch.bfloat16))
    assert np.array_equal(f.view(np.uint32), orc.dequant_f32(w, rows, cols).view(np.uint32))
    assert np.array_equal(b, orc.dequant_bf16(w, rows, cols))


def test_full_size_bitwise(m, orc):
    rows, cols = 14336, 4096
    w, _ = inputs.gemm_case(3, rows, cols, 1)
    f = host(m.mxfp4_dequant(dev(w), rows, cols, out_dtype=torch.float32))
    assert np.array_equal(f.view(np.uint32), orc.dequant_f32(w, rows, cols).view(np.uint32))


def test_guard_band(m, orc):
    """Writes stay inside the output (canaries on both sides)."""
    rows, cols = 7, 96
    w, _ = inputs.gemm_case(4, rows, cols, 1)
    buf = torch.full((rows * cols + 64,), 12345.0, device="cuda")
    out = buf[32:32 + rows * cols]
    m.mxfp4_dequant(dev(w), rows, cols, out=out)
    hb = host(buf)
    assert np.all(hb[:32] == 12345.0) and np.all(hb[-32:] == 12345.0)
    assert np.array_equal(hb[32:-32].view(np.uint32),
                          orc.dequant_f32(w, rows, cols).reshape(-1).view(np.uint32))
