"""GPU parity of the opt-in FP4 x FP8 expert bank (moe_experts_mxfp4_a8).

Reference: the oracle's expert bank with the same two quantizations the
entry point applies, composed from oracle functions only: x -> MXFP8
(mxfp8_quantize, bit-exact against the GPU's quantizer in test_gpu_mx8),
gate/up and SwiGLU in fp64, h rounded to fp32 (the GPU keeps h in fp32)
and quantized to MXFP8, down, the weighted sum in slot order, out rounded
to bf16.  Tolerance: the MoE-frame check of "cortiq-engine 0.8.40,
src/gpu_wgpu/mxfp4.rs" (global_bank_frame tests: nrmse < 0.01 at release
geometry, cosine > 0.999) over every checked token.  What separates the two
sides: the matrix core's in-block accumulation (within 2^-7 of sum |w * a|
per product by the entry point's contract), a rare E4M3 step where the
GPU's fp32 h and the oracle's h straddle a rounding boundary, and the bf16
output rounding; a wrong expert, slot or permutation gives nrmse near 1.
"""
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


def x_f64(c, xd):
    x = c["x"]
    return bf16_to_f64(x) if xd == "bf16" else np.asarray(x, np.float64)


def oracle_out(orc, c, E, H, I, xd, ids, dense=False):
    """bf16-rounded fp64 output of the quantizing bank for routing ``ids``
    (pairs with id -1 dropped)."""
    xq = orc.mxfp8_dequantize(*orc.mxfp8_quantize(x_f64(c, xd)))
    gate_up = orc.moe_gate_up_dense if dense else orc.moe_gate_up
    down = orc.moe_down_dense if dense else orc.moe_down
    st = gate_up(c["gate"], c["up"], E, H, I, xq, ids, False)
    hq = orc.mxfp8_dequantize(*orc.mxfp8_quantize(st["h"].astype(np.float32)))
    y, mag_y = down(c["down"], E, H, I, hq, ids)
    out, _ = orc.moe_combine(y, mag_y, c["w"], ids, E)
    return bf16_to_f64(orc.bf16_rne_array(out).reshape(out.shape))


def gpu_out(m, c, E, H, I):
    d = {k: dev(v) for k, v in c.items()}
    out = m.moe_experts_mxfp4_a8(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                 d["w"])
    torch.cuda.synchronize()
    return bf16_to_f64(host(out))


def assert_frame(got, ref, what):
    assert np.isfinite(got).all() and np.isfinite(ref).all(), what
    nrmse = np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    cos = float((got * ref).sum() / np.sqrt((got * got).sum() * (ref * ref).sum()))
    assert nrmse < 0.01 and cos > 0.999, (what, nrmse, cos)
    return nrmse, cos


@pytest.mark.parametrize("E,H,I,T,K,xd,routing", [
    (8, 512, 512, 24, 2, "bf16", "softmax"),    # one item per expert, ragged tokens
    (16, 1024, 512, 100, 4, "f32", "zipf"),     # hot experts over several 64-token items
    (6, 512, 1536, 70, 3, "bf16", "zipf"),      # 3-unit down K, 12 gate/up row blocks
    (40, 1024, 1024, 13, 5, "f32", "softmax"),  # few tokens per expert
])
def test_bank_against_quantizing_oracle(m, orc, E, H, I, T, K, xd, routing):
    c = inputs.moe_case(E * 1000 + T, E, H, I, T, K, xd, routing, scale_lo=100, scale_hi=114)
    got = gpu_out(m, c, E, H, I)
    ref = oracle_out(orc, c, E, H, I, xd, c["ids"])
    assert_frame(got, ref, f"a8 bank E={E} H={H} I={I} T={T} K={K} {xd} {routing}")


def test_dropped_pairs(m, orc):
    E, H, I, T, K = 8, 512, 512, 20, 3
    c = inputs.moe_case(49, E, H, I, T, K, "bf16", "softmax", scale_lo=100, scale_hi=114)
    c["ids"] = c["ids"].copy()
    c["ids"][2, 1] = -1
    c["ids"][7, 0] = E + 3
    got = gpu_out(m, c, E, H, I)
    ref = oracle_out(orc, c, E, H, I, "bf16", c["ids"])
    assert_frame(got, ref, "dropped pairs")


def test_token_alone_equals_batch_bitwise(m):
    """A token's output is the same bits alone or in a batch: its column of
    every product, its quantization blocks and its slot sum depend on it
    alone."""
    E, H, I, T, K = 6, 1024, 512, 90, 3
    c = inputs.moe_case(50, E, H, I, T, K, "bf16", "zipf", scale_lo=100, scale_hi=114)
    d = {k: dev(v) for k, v in c.items()}
    full = host(m.moe_experts_mxfp4_a8(d["gate"], d["up"], d["down"], E, H, I, d["x"],
                                       d["ids"], d["w"]))
    for t in (0, 37, T - 1):
        one = host(m.moe_experts_mxfp4_a8(d["gate"], d["up"], d["down"], E, H, I,
                                          d["x"][t:t + 1].contiguous(),
                                          d["ids"][t:t + 1].contiguous(),
                                          d["w"][t:t + 1].contiguous()))
        assert np.array_equal(one[0].view(np.uint16), full[t].view(np.uint16)), t
    again = host(m.moe_experts_mxfp4_a8(d["gate"], d["up"], d["down"], E, H, I, d["x"],
                                        d["ids"], d["w"]))
    assert np.array_equal(again.view(np.uint16), full.view(np.uint16))


def test_prefill_layer_sampled(m, orc, prefill_case):
    """The 256-expert prefill layer at full size on the GPU; the oracle on 8
    tokens (their pairs only), dense form."""
    cfg = inputs.WORKLOADS[5]
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
    c = prefill_case
    got = gpu_out(m, c, E, H, I)
    T = c["ids"].shape[0]
    toks = np.array([0, 1, 100, 255, 256, 400, 510, T - 1])
    ids = np.full_like(c["ids"], -1)
    ids[toks] = c["ids"][toks]
    ref = oracle_out(orc, c, E, H, I, cfg["x_dtype"], ids, dense=True)
    assert_frame(got[toks], ref[toks], "prefill layer, 8 tokens")
