"""The Python binding refuses host tensors before anything reaches the
library (no GPU needed): the C ABI takes raw device pointers, so a host
pointer passed through would be dereferenced by a kernel.  The checks of
strides, element types and buffer lengths, which need device tensors, are
in test_gpu_binding.py."""
import os

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gemm_mxfp4_dequant_amd", "libmxfp4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmxfp4.so not built")


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def _w(rows, cols, n=1):
    return torch.zeros(n * (rows * cols // 2 + rows * cols // 32), dtype=torch.uint8)


def test_host_tensors_refused(m):
    rows, cols, b = 64, 512, 2
    w = _w(rows, cols)
    x = torch.zeros((b, cols))
    cases = [
        lambda: m.mxfp4_dequant(w, rows, cols),
        lambda: m.mxfp4_matvec(w, rows, cols, x[0]),
        lambda: m.mxfp4_gemm(w, rows, cols, x),
        lambda: m.moe_route_group(torch.zeros((2, 2), dtype=torch.int32), 4),
        lambda: m.moe_route_topk(torch.zeros((2, 8)), 2),
    ]
    E, H, I, T, K = 4, 512, 256, 3, 2
    bank = _w(I, H, E)
    down = _w(H, I, E)
    ids = torch.zeros((T, K), dtype=torch.int32)
    wr = torch.full((T, K), 0.5)
    xm = torch.zeros((T, H))
    cases += [
        lambda: m.moe_experts_mxfp4(bank, bank, down, E, H, I, xm, ids, wr),
        lambda: m.moe_experts_mxfp4_stages(bank, bank, down, E, H, I, xm, ids, wr,
                                           h_out=torch.zeros((T * K, I))),
        lambda: m.moe_experts_mxfp4_v41(bank, bank, down, E, H, I, xm.bfloat16(), ids, wr),
        lambda: m.moe_experts_mxfp4_v41_stages(bank, bank, down, E, H, I, xm.bfloat16(), ids,
                                               wr, h_out=torch.zeros((T * K, I),
                                                                     dtype=torch.bfloat16)),
    ]
    for i, f in enumerate(cases):
        with pytest.raises(ValueError, match="device"):
            f()


def test_non_tensor_and_bad_sizes_refused(m):
    with pytest.raises(TypeError):
        m.mxfp4_gemm(np.zeros(10, np.uint8), 16, 64, torch.zeros((1, 64)))
    with pytest.raises(TypeError):
        m.mxfp4_gemm(_w(16, 64), 16.0, 64, torch.zeros((1, 64)))
    with pytest.raises(ValueError, match="MXFP4 shape"):
        m.mxfp4_dequant(torch.zeros(100, dtype=torch.uint8), 4, 48)
