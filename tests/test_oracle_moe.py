"""Pins for the oracle's routed expert bank.

* grouping: against Python's stable ``sorted`` of the pairs by expert;
* SwiGLU: the identity silu(g) - silu(-g) = g, exercised by negating every
  gate weight (sign bit of each nibble), plus silu(0) = 0;
* the whole bank: against an independent fp64 computation on tiny shapes
  whose weights come from the E2M1 field definition and whose products are
  numpy matmuls;
* invariants: identical experts with weights summing to 1 make the output
  independent of the routing; scaling the route weights scales the output.
Semantics follow "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs"
(gate_up_block, down_block) and "cortiq-engine 0.8.40,
src/gpu_wgpu/mxfp4.rs" (dsv4_global_down_mxfp4, generic f32 weighting).
"""
import numpy as np
import pytest

from gemm_mxfp4_dequant_amd import inputs


def tensor_values(w, rows, cols):
    """fp64 weights from the field definition (independent of the oracle)."""
    cb = w[: rows * cols // 2].astype(np.int64)
    codes = np.empty(rows * cols, np.int64)
    codes[0::2] = cb & 15
    codes[1::2] = cb >> 4
    s = (codes >> 3) & 1
    e = (codes >> 1) & 3
    m = codes & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1 + m * 0.5))
    sc = w[rows * cols // 2: rows * cols // 2 + rows * cols // 32].astype(np.float64)
    v = np.where(s == 1, -mag, mag) * np.repeat(np.exp2(sc - 127), 32)
    return v.reshape(rows, cols)


def small_case(seed, E=5, H=64, I=96, T=4, K=2, xd="f32", lo=112, hi=120):
    c = inputs.moe_case(seed, E, H, I, T, K, xd, "softmax", scale_lo=lo, scale_hi=hi)
    return c, E, H, I, T, K


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_group_matches_stable_sort(orc, seed):
    rng = np.random.default_rng(seed)
    E = 13
    ids = rng.integers(0, E, size=(37, 3)).astype(np.int32)
    ids[3, 1] = -1
    ids[5, 0] = E + 2  # out of range: left out
    counts, offsets, pos, slot = orc.group(ids, E)
    flat = ids.reshape(-1)
    valid = [p for p in range(flat.size) if 0 <= flat[p] < E]
    order = sorted(valid, key=lambda p: flat[p])  # Python's sort is stable
    assert list(pos) == order
    for e in range(E):
        assert counts[e] == sum(1 for p in valid if flat[p] == e)
        assert offsets[e + 1] - offsets[e] == counts[e]
    for s, p in enumerate(order):
        assert slot[p] == s
    assert slot[3 * 3 + 1] == -1 and slot[5 * 3] == -1


@pytest.mark.parametrize("xd,round_h", [("f32", False), ("bf16", True)])
def test_bank_matches_independent_fp64(orc, xd, round_h):
    c, E, H, I, T, K = small_case(3, xd=xd)
    res = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"], c["w"], round_h)
    x = orc._as_f64(c["x"])
    gb, db = inputs.tensor_nbytes(I, H), inputs.tensor_nbytes(H, I)
    out = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = int(c["ids"][t, k])
            Wg = tensor_values(c["gate"][e * gb:(e + 1) * gb], I, H)
            Wu = tensor_values(c["up"][e * gb:(e + 1) * gb], I, H)
            Wd = tensor_values(c["down"][e * db:(e + 1) * db], H, I)
            g = Wg @ x[t]
            u = Wu @ x[t]
            h = g / (1 + np.exp(-g)) * u
            p = t * K + k
            np.testing.assert_allclose(res["g"][p], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
            np.testing.assert_allclose(res["u"][p], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
            if round_h:
                h = orc.bf16_bits_to_f64(orc.bf16_rne_array(h))
                # a tie-near value could round the other way; allow one bf16 ulp
                np.testing.assert_allclose(res["h"][p], h, rtol=2 ** -7)
            else:
                np.testing.assert_allclose(res["h"][p], h, rtol=1e-11, atol=1e-11 * np.abs(h).max())
            y = Wd @ res["h"][p]
            np.testing.assert_allclose(res["y"][p], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
            out[t] += float(c["w"][t, k]) * y
    np.testing.assert_allclose(res["out"], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())
    assert np.array_equal(res["out_bf16"], orc.bf16_rne_array(res["out"]).reshape(T, H))


def test_swiglu_odd_identity(orc):
    """Negating all gate weights negates g; silu(g) - silu(-g) = g, so
    h(W_g) - h(-W_g) = g * u."""
    c, E, H, I, T, K = small_case(4, lo=118, hi=124)
    a = orc.moe_gate_up(c["gate"], c["up"], E, H, I, c["x"], c["ids"], False)
    neg = c["gate"].copy()
    gb = inputs.tensor_nbytes(I, H)
    for e in range(E):
        neg[e * gb: e * gb + I * H // 2] ^= 0x88
    b = orc.moe_gate_up(neg, c["up"], E, H, I, c["x"], c["ids"], False)
    assert np.array_equal(b["g"], -a["g"])
    lhs = a["h"] - b["h"]
    rhs = a["g"] * a["u"]
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12 * np.abs(rhs).max())


def test_zero_gate_gives_zero_h(orc):
    c, E, H, I, T, K = small_case(5)
    zg = c["gate"].copy()
    gb = inputs.tensor_nbytes(I, H)
    for e in range(E):
        zg[e * gb: e * gb + I * H // 2] = 0
    st = orc.moe_gate_up(zg, c["up"], E, H, I, c["x"], c["ids"], False)
    assert np.all(st["g"] == 0) and np.all(st["h"] == 0)


def test_identical_experts_routing_invariant(orc):
    c, E, H, I, T, K = small_case(6, E=4, K=3)
    gb, db = inputs.tensor_nbytes(I, H), inputs.tensor_nbytes(H, I)
    for key, nb in (("gate", gb), ("up", gb), ("down", db)):
        c[key] = np.tile(c[key][:nb], E)
    r1 = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"], c["w"], False)
    ids2 = np.roll(c["ids"], 1, axis=1)
    ids2 = (ids2 + 1) % E
    w2 = np.full_like(c["w"], 1.0 / K)
    r2 = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], ids2, w2, False)
    ref = r1["y"].reshape(T, K, H)[:, 0, :]  # one expert's output per token
    scale = np.abs(ref).max()
    np.testing.assert_allclose(r1["out"] / c["w"].astype(np.float64).sum(1, keepdims=True),
                               ref, rtol=1e-6, atol=1e-9 * scale)
    np.testing.assert_allclose(r2["out"] * (1.0 / (K * np.float32(1.0 / K))), ref,
                               rtol=1e-6, atol=1e-9 * scale)


def test_weights_scale_output(orc):
    c, E, H, I, T, K = small_case(8)
    r1 = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"], c["w"], False)
    r2 = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"], c["w"] * 2, False)
    assert np.array_equal(r2["out"], 2 * r1["out"])
    assert np.array_equal(r2["mag_out"], 2 * r1["mag_out"])


@pytest.mark.parametrize("xd,round_h", [("f32", False), ("bf16", True), ("bf16", False)])
def test_dense_form_equals_loop_form(orc, xd, round_h):
    """The dense form of the expert stages (each expert dequantized once,
    fp64 matrix products) against the loop form, which the tests above pin:
    g, u, y and their magnitudes within fp64 rounding of the magnitude sums,
    h (and its bf16 rounding) alike, dropped pairs zero in both, NaN rows
    where a scale byte is 255."""
    E, H, I, T, K = 6, 256, 160, 9, 3
    c = inputs.moe_case(301, E, H, I, T, K, xd, "softmax", scale_lo=100, scale_hi=130)
    ids = c["ids"].copy()
    ids[2, 1] = -1
    ids[5, 0] = E + 2
    nb = orc.nbytes(I, H)
    gate = c["gate"].copy()
    gate[2 * nb + I * H // 2 + 3 * (H // 32) + 1] = 255   # expert 2, row 3, group 1
    lf = orc.moe_gate_up(gate, c["up"], E, H, I, c["x"], ids, round_h)
    df = orc.moe_gate_up_dense(gate, c["up"], E, H, I, c["x"], ids, round_h)
    # each quantity within 1e-12 of its own magnitude sum (fp64 rounding of
    # sums in a different order); h through silu(g) u of those
    scales = {"g": lf["mag_g"], "u": lf["mag_u"], "mag_g": lf["mag_g"], "mag_u": lf["mag_u"],
              "h": lf["mag_g"] * np.abs(lf["u"]) + lf["mag_u"] + np.abs(lf["h"])}
    for k in ("g", "u", "h", "mag_g", "mag_u"):
        a, b = lf[k], df[k]
        assert np.array_equal(np.isnan(a), np.isnan(b)), k
        ok = ~np.isnan(a)
        assert np.all(np.abs(a[ok] - b[ok]) <= 1e-12 * scales[k][ok] + 1e-300), k
    assert np.isnan(lf["g"]).any() and not np.isnan(lf["u"]).any()
    assert np.all(df["g"][[2 * K + 1, 5 * K + 0]] == 0)
    if round_h:
        fin = np.isfinite(lf["h"])
        assert np.array_equal(lf["h"][fin], df["h"][fin])
    h = np.where(np.isnan(lf["h"]), 0.0, lf["h"])
    y1, m1 = orc.moe_down(c["down"], E, H, I, h, ids)
    y2, m2 = orc.moe_down_dense(c["down"], E, H, I, h, ids)
    assert np.all(np.abs(y1 - y2) <= 1e-12 * m1 + 1e-300)
    assert np.all(np.abs(m1 - m2) <= 1e-12 * m1 + 1e-300)


def test_dense_form_refuses_overflowing_weights(orc):
    """Scale 254 with |code| >= 2 overflows fp32: the dense form (built on
    the fp32 dequantization) refuses rather than return inf products."""
    E, H, I, T, K = 2, 64, 32, 2, 1
    c = inputs.moe_case(302, E, H, I, T, K, "f32", "softmax", scale_lo=254, scale_hi=254)
    with pytest.raises(AssertionError, match="overflows"):
        orc.moe_gate_up_dense(c["gate"], c["up"], E, H, I, c["x"], c["ids"], False)
