"""Pins for the oracle's V4.1 expert bank (bf16 gate/up, SwiGLU limit,
route weight folded into a bf16 activation, one bf16 rounding of the summed
down outputs, optional shared expert): "cortiq-engine 0.8.40,
src/gpu_wgpu/mxfp4.rs", dsv4_global_gate_up_mxfp4 / dsv4_global_down_mxfp4
with their bf16 flag, and the host expert of global_bank_case.

Each pin compares the oracle with something other than its own formula:
hand-worked values, the already-pinned bf16 SwiGLU of the plain bank, and
exact invariants of the definition."""
import numpy as np
import pytest

from gemm_mxfp4_dequant_amd import inputs


def one_hot_case(cols, rows, codes_scales, hot):
    """A weight tensor whose row r holds one nonzero code at column `hot`
    (code, scale from codes_scales[r]); every other code is 0 (+0)."""
    codes = np.zeros(rows * cols // 2, np.uint8)
    scales = np.full(rows * cols // 32, 127, np.uint8)
    for r, (code, scale) in enumerate(codes_scales):
        b = (r * cols + hot) // 2
        codes[b] |= (code << 4) if hot & 1 else code
        scales[r * (cols // 32) + hot // 32] = scale
    return np.concatenate([codes, scales])


def test_exact_gate_up_reduces_to_bf16_swiglu(orc):
    """With gate/up products exactly representable in bf16, no limit and
    weight 1, the V4.1 activation is the plain bank's bf16-rounded SwiGLU."""
    H, I = 64, 8
    cs_g = [(c, s) for c, s in zip([1, 2, 3, 9, 12, 7, 5, 14], [127, 126, 128, 129, 125, 127, 130, 124])]
    cs_u = [(c, s) for c, s in zip([6, 3, 11, 2, 4, 15, 13, 1], [128, 127, 126, 129, 127, 125, 127, 128])]
    gate = one_hot_case(H, I, cs_g, 5)
    up = one_hot_case(H, I, cs_u, 5)
    x = np.zeros((1, H), np.float32)
    x[0, 5] = 1.0
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    plain = orc.moe_gate_up(gate, up, 1, H, I, x, ids, True)
    exact = orc.moe_gate_up(gate, up, 1, H, I, x, ids, False)
    h = orc.moe_v41_act(exact["g"], exact["u"], w, ids, 1, 0.0)
    assert np.array_equal(h, plain["h"])


def test_limit_worked_by_hand(orc):
    """gate 12 -> capped at 10; up -24 -> clamped to -10; gate -12 is not
    raised (the gate has no lower bound); weight 0.5.
    h = bf16(0.5 * silu(10) * -10) = bf16(-49.99773) = -50 (bf16 spacing
    0.25 in [32, 64)); h = bf16(0.5 * silu(-12) * -10) with
    silu(-12) = -12 / (1 + e^12) = -7.3730e-5, so 0.5 * -7.3730e-5 * -10 =
    3.68650e-4, in [2^-12, 2^-11) where the bf16 spacing is 2^-19:
    3.68650e-4 / 2^-19 = 193.27 -> 193 * 2^-19."""
    g = np.array([[12.0, -12.0]])
    u = np.array([[-24.0, -24.0]])
    ids = np.zeros((1, 1), np.int32)
    h = orc.moe_v41_act(g, u, np.array([[0.5]]), ids, 1, 10.0)
    assert h[0, 0] == -50.0
    assert h[0, 1] == 193 * 2.0 ** -19
    # the limit only acts when positive: 0.5 * silu(12) * -24 = -143.99918,
    # bf16 spacing 1 in [128, 256) -> -144
    h0 = orc.moe_v41_act(g, u, np.array([[0.5]]), ids, 1, 0.0)
    assert h0[0, 0] == -144.0


def test_power_of_two_weights_scale_exactly(orc):
    rng = np.random.default_rng(3)
    g = rng.normal(size=(4, 64)) * 3
    u = rng.normal(size=(4, 64)) * 3
    ids = np.zeros((1, 4), np.int32)
    h1 = orc.moe_v41_act(g, u, np.ones((1, 4)), ids, 1, 6.0)
    for wv in (0.5, 0.25, 2.0, -0.125):
        hw = orc.moe_v41_act(g, u, np.full((1, 4), wv), ids, 1, 6.0)
        assert np.array_equal(hw, wv * h1)


def test_two_half_slots_equal_one_full_slot(orc):
    """The route weight is folded into h before the down product and the
    down outputs are summed unweighted: one expert taken twice with weight
    1/2 gives the same out as once with weight 1 (all steps exact in fp64)."""
    E, H, I, T = 3, 64, 32, 4
    c = inputs.moe_case(71, E, H, I, T, 1, "bf16", "softmax", scale_lo=110, scale_hi=125)
    ids1 = c["ids"][:, :1].copy()
    w1 = np.ones((T, 1), np.float32)
    ids2 = np.repeat(ids1, 2, axis=1)
    w2 = np.full((T, 2), 0.5, np.float32)
    a = orc.moe_v41(c["gate"], c["up"], c["down"], E, H, I, c["x"], ids1, w1, 4.0, False)
    b = orc.moe_v41(c["gate"], c["up"], c["down"], E, H, I, c["x"], ids2, w2, 4.0, False)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["out_bf16"], b["out_bf16"])


def test_shared_expert_is_one_more_slot(orc):
    """has_shared adds expert E to every token with weight 1: the same as
    routing it explicitly (banks of E + 1 experts)."""
    E, H, I, T, K = 4, 64, 32, 5, 2
    c = inputs.moe_case(72, E + 1, H, I, T, K, "bf16", "softmax", scale_lo=110, scale_hi=125)
    ids = np.minimum(c["ids"], E - 1).astype(np.int32)
    ids[1, 0] = -1  # a dropped pair stays dropped
    a = orc.moe_v41(c["gate"], c["up"], c["down"], E, H, I, c["x"], ids, c["w"], 7.0, True)
    ids_x = np.concatenate([ids, np.full((T, 1), E, np.int32)], axis=1)
    w_x = np.concatenate([c["w"], np.ones((T, 1), np.float32)], axis=1)
    b = orc.moe_v41(c["gate"], c["up"], c["down"], E + 1, H, I, c["x"], ids_x, w_x, 7.0, False)
    assert np.array_equal(a["out_bf16"], b["out_bf16"])
    assert np.array_equal(a["h"], b["h"])


def test_out_is_bf16_of_the_slot_sum(orc):
    """out_bf16 is the one rounding of the fp64 sum of the slots' down
    outputs; every h is a bf16 value."""
    E, H, I, T, K = 4, 64, 32, 3, 3
    c = inputs.moe_case(73, E, H, I, T, K, "bf16", "softmax", scale_lo=110, scale_hi=125)
    r = orc.moe_v41(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"], c["w"], 0.0, False)
    hb = orc.bf16_bits_to_f64(orc.bf16_rne_array(r["h"])).reshape(r["h"].shape)
    assert np.array_equal(hb, r["h"])
    s = r["y"].reshape(T, K, H).sum(axis=1)
    assert np.allclose(s, r["out"], rtol=0, atol=1e-12 * np.abs(r["y"]).max())
