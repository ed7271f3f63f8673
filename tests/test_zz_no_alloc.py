"""The allocation-free expert bank (moe_experts_mxfp4_noalloc: the static
device scratch instead of a caller workspace) against moe_experts_mxfp4 with
a workspace, through the C ABI: the same kernels in the same order, so the
outputs must be equal bit for bit.  Two calls in a row on the one static
scratch, the second with fewer tokens (and then the first again), so a call
that read anything the previous call left behind would differ.  The first
bank's output is also checked against the oracle (end-to-end nrmse / cos,
as the expert-bank tests do)."""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import bf16_to_f64, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def upload(c):
    return {k: dev(v) for k, v in c.items()}


def with_ws(m, d, E, H, I):
    return host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                    d["w"]))


def no_alloc(m, d, E, H, I):
    T = d["ids"].shape[0]
    out = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
    m.moe_experts_mxfp4_noalloc(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                d["w"], out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("xd,shape", [("f32", "decode"), ("bf16", "decode"), ("bf16", "tiled")])
def test_noalloc_equals_workspace_bank(m, orc, xd, shape):
    # decode: 48 pairs on 16 experts (split-K kernels, grouping inside
    # gate/up); tiled: 192 Zipf-routed pairs (tiled kernels, with experts
    # of at most four pairs on the skinny down kernel)
    if shape == "decode":
        E, H, I, T, K, routing, t_small = 16, 4096, 2048, 8, 6, "softmax", 3
    else:
        E, H, I, T, K, routing, t_small = 16, 1024, 512, 96, 2, "zipf", 40
    big = inputs.moe_case(61, E, H, I, T, K, xd, routing, scale_lo=100, scale_hi=114)
    if shape == "tiled":
        cnt = np.bincount(big["ids"].reshape(-1), minlength=E)
        assert cnt.max() > 16 and ((cnt > 0) & (cnt <= 4)).any(), cnt
    small = dict(big)
    small["x"], small["ids"], small["w"] = (big["x"][:t_small], big["ids"][:t_small],
                                            big["w"][:t_small])
    db, ds = upload(big), upload(small)
    ref_b, ref_s = with_ws(m, db, E, H, I), with_ws(m, ds, E, H, I)
    got_b = no_alloc(m, db, E, H, I)
    got_s = no_alloc(m, ds, E, H, I)
    got_b2 = no_alloc(m, db, E, H, I)
    assert np.array_equal(got_b, ref_b), "first call"
    assert np.array_equal(got_s, ref_s), "second, smaller call"
    assert np.array_equal(got_b2, ref_b), "the first shape again"
    # and the bank itself against the oracle (both sides rounded to bf16)
    ref = orc.moe(big["gate"], big["up"], big["down"], E, H, I, big["x"], big["ids"], big["w"],
                  xd == "bf16")
    want = bf16_to_f64(ref["out_bf16"])
    got = bf16_to_f64(got_b)
    nrmse = np.sqrt(np.mean((got - want) ** 2)) / np.sqrt(np.mean(want ** 2))
    cos = float((got * want).sum() / np.sqrt((got * got).sum() * (want * want).sum()))
    assert nrmse < 1e-3 and cos > 0.9999, (nrmse, cos)


def test_noalloc_refuses_sizes_beyond_the_scratch(m):
    """A bank whose workspace would exceed the static scratch is refused
    before any launch, and the output is left untouched."""
    E, H, I, T, K = 4, 4096, 512, 1024, 4   # y alone: 4096 pairs x 4096 x 4 B = 64 MiB
    need = m.moe_experts_mxfp4_workspace_size(T, K, E, H, I, torch.float32)
    assert need > m.MXFP4_NOALLOC_SCRATCH_BYTES
    nb = I * H // 2 + I * H // 32
    bank = torch.zeros(E * nb, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    w = torch.full((T, K), 0.25, device="cuda")
    x = torch.zeros((T, H), device="cuda")
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.Mxfp4Error) as e:
        m.moe_experts_mxfp4_noalloc(bank, bank, bank, E, H, I, x, ids, w, out)
    assert e.value.status == m.MXFP4_EWORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_noalloc_at_the_scratch_cap(m):
    """The largest routing whose scratch fits MXFP4_NOALLOC_SCRATCH_BYTES (16
    experts of 4096 x 2048, Zipf top 8, fp32; the token count found with the
    size query) gives the workspace call's bits; one token more is refused
    before any launch."""
    E, H, I, K = 16, 4096, 2048, 8
    cap = m.MXFP4_NOALLOC_SCRATCH_BYTES

    def need(T):
        return m.moe_experts_mxfp4_workspace_size(T, K, E, H, I, torch.float32)

    lo, hi = 1, 1 << 20
    while lo < hi:  # the largest T with need(T) <= cap
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if need(mid) <= cap else (lo, mid - 1)
    T = lo
    assert need(T) <= cap < need(T + 1)
    c = inputs.moe_case(62, E, H, I, T, K, "f32", "zipf", scale_lo=100, scale_hi=114)
    d = upload(c)
    assert np.array_equal(no_alloc(m, d, E, H, I), with_ws(m, d, E, H, I)), T
    x1 = torch.zeros((T + 1, H), device="cuda")
    ids1 = torch.zeros((T + 1, K), dtype=torch.int32, device="cuda")
    w1 = torch.full((T + 1, K), 0.125, device="cuda")
    out1 = torch.full((T + 1, H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.Mxfp4Error) as e:
        m.moe_experts_mxfp4_noalloc(d["gate"], d["up"], d["down"], E, H, I, x1, ids1, w1, out1)
    assert e.value.status == m.MXFP4_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out1 == 3.0)
