"""GPU parity of the V4.1 expert bank (moe_experts_mxfp4_v41) against the
oracle: bf16 gate/up, SwiGLU limit, route weight folded into the bf16
activation, slots summed unweighted and rounded once, optional shared
expert ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs": dsv4_global_gate_up_
mxfp4 / dsv4_global_down_mxfp4 with their bf16 flag, and the host expert of
global_bank_case).

* stage isolation, h (slot order) against the oracle's h:
    |h_gpu - h_or| <= |w| (1.1 dg |u_b| + |silu(g_b)| du) + 1 ulp_bf16(h_or)
  with dg = 1e-4 mag_g + ulp_bf16(g), du = 1e-4 mag_u + ulp_bf16(u): the
  library's product rule plus one bf16 step of g or u (both sides round
  their own sums to bf16), through silu (|silu'| < 1.1) and the clamp
  (1-Lipschitz), then h's own rounding;
* down + combine fed with h_gpu:
    |out_gpu - out_or| <= 1e-4 sum_k mag_y + 1 ulp_bf16(out_or);
* end to end: nrmse < 2e-3 and cosine > 0.9999 against the oracle's bf16
  output (the pages' own bank check allows nrmse 0.01-0.02, cos > 0.999);
* invariants: a token alone equals the batch bit for bit; routed ids equal
  to n_experts never reach the shared expert.
"""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import assert_within, bf16_to_f64, dev, host, ulp_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def bank_case(seed, E, H, I, T, K, shared, routing="softmax", lo=110, hi=125):
    """Inputs with banks of E (+1 shared) experts; bf16 activations."""
    c = inputs.moe_case(seed, E + int(shared), H, I, T, K, "bf16", routing,
                        scale_lo=lo, scale_hi=hi)
    ids = c["ids"].copy()
    ids[ids >= E] = ids[ids >= E] % E  # routed ids stay below E
    c["ids"] = ids.astype(np.int32)
    return c


def run(m, d, E, H, I, lim, shared, **kw):
    return m.moe_experts_mxfp4_v41(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                   d["w"], swiglu_limit=lim, has_shared=shared, **kw)


def check(m, orc, c, E, H, I, lim, shared, tokens=None, pairs=None, e2e_tokens=None,
          dense=False):
    """h for the augmented-routing pairs ``pairs`` (default: every pair of
    ``tokens``, or of all tokens), down + combine for ``tokens``, end to end
    for ``e2e_tokens`` (default: ``tokens``).  ``dense``: the oracle's
    gate/up in its dense form."""
    T, K = c["ids"].shape
    d = {k: dev(v) for k, v in c.items()}
    ids_a, w_a, Ea = orc.v41_routing(c["ids"], c["w"], E, shared)
    Ka = ids_a.shape[1]
    Pa = T * Ka
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    keep = np.zeros(T, bool)
    keep[tok] = True
    ids_k = np.where(keep[:, None], ids_a, -1).astype(np.int32)
    if pairs is None:
        ids_h = ids_k
    else:
        flat = np.full(Pa, -1, np.int32)
        flat[pairs] = ids_a.reshape(-1)[pairs]
        ids_h = flat.reshape(T, Ka)

    # stage isolation: h in slot order of the augmented routing
    h = torch.empty((Pa, I), dtype=torch.bfloat16, device="cuda")
    m.moe_experts_mxfp4_v41_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                   d["w"], swiglu_limit=lim, has_shared=shared, h_out=h)
    _, _, slot = m.moe_route_group(dev(ids_a), Ea)
    slot = host(slot)
    h_gpu = host(h)
    gate_up = orc.moe_gate_up_dense if dense else orc.moe_gate_up
    st = gate_up(c["gate"], c["up"], Ea, H, I, c["x"], ids_h, False)
    h_or = orc.moe_v41_act(st["g"], st["u"], w_a, ids_h, Ea, lim)
    flat = ids_h.reshape(-1)
    valid = np.where((flat >= 0) & (flat < Ea))[0]
    hp = bf16_to_f64(h_gpu[slot[valid]])
    g, u = st["g"][valid], st["u"][valid]
    gb = bf16_to_f64(orc.bf16_rne_array(g)).reshape(g.shape)
    ub = bf16_to_f64(orc.bf16_rne_array(u)).reshape(u.shape)
    if lim > 0:
        ub = np.clip(ub, -lim, lim)
        gb = np.minimum(gb, lim)
    wv = np.abs(w_a.reshape(-1)[valid])[:, None]
    dg = 1e-4 * st["mag_g"][valid] + ulp_bf16(g)
    du = 1e-4 * st["mag_u"][valid] + ulp_bf16(u)
    silu_b = gb / (1.0 + np.exp(-np.clip(gb, -700, 700)))
    bound = wv * (1.1 * dg * np.abs(ub) + np.abs(silu_b) * du)
    # the bound is absolute (already holds the 1e-4 product rule)
    assert_within(hp, h_or[valid], np.zeros_like(bound), extra=bound + ulp_bf16(h_or[valid]),
                  what="h (V4.1)")

    # down + combine fed with the device h
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    m.moe_experts_mxfp4_v41_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                   d["w"], swiglu_limit=lim, has_shared=shared, out=out,
                                   h_in=dev(h_gpu))
    out_g = bf16_to_f64(host(out))
    h_pair = np.zeros((Pa, I))
    vv = np.where(slot >= 0)[0]
    h_pair[vv] = bf16_to_f64(h_gpu[slot[vv]])
    y, mag_y = orc.moe_down(c["down"], Ea, H, I, h_pair, ids_k)
    o, mag_o = orc.moe_combine(y, mag_y, np.ones(ids_k.shape), ids_k, Ea)
    assert_within(out_g[tok], o[tok], mag_o[tok], extra=ulp_bf16(o[tok]), what="down+combine")

    # end to end against the oracle's own chain
    te = tok if e2e_tokens is None else np.asarray(e2e_tokens)
    out2 = bf16_to_f64(host(run(m, d, E, H, I, lim, shared)))
    ref = orc.moe_v41(c["gate"], c["up"], c["down"], E, H, I, c["x"][te], c["ids"][te],
                      c["w"][te], lim, shared)
    ref = bf16_to_f64(ref["out_bf16"])
    got = out2[te]
    nrmse = np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    cos = float((got * ref).sum() / np.sqrt((got * got).sum() * (ref * ref).sum()))
    assert nrmse < 2e-3 and cos > 0.9999, (nrmse, cos)
    return out2


@pytest.mark.parametrize("lim", [0.0, 1.5])
@pytest.mark.parametrize("shared", [False, True])
def test_small_bank(m, orc, lim, shared):
    """Few tokens per expert (skinny kernels); the limit clamps many values."""
    E, H, I, T, K = 8, 512, 256, 9, 3
    check(m, orc, bank_case(80 + int(shared), E, H, I, T, K, shared), E, H, I, lim, shared)


@pytest.mark.parametrize("shared", [False, True])
def test_many_tokens_per_expert(m, orc, shared):
    """Tens of tokens per expert (tiled kernels), ragged column tiles."""
    E, H, I, T, K = 4, 1024, 512, 90, 2
    check(m, orc, bank_case(84, E, H, I, T, K, shared), E, H, I, 2.0, shared)


def test_dropped_ids_never_reach_the_shared_expert(m, orc):
    E, H, I, T, K = 6, 512, 256, 7, 2
    c = bank_case(86, E, H, I, T, K, True)
    c["ids"][1, 0] = -1
    c["ids"][2, 1] = E       # the shared expert's index: must be dropped
    c["ids"][4, 0] = E + 40
    check(m, orc, c, E, H, I, 1.0, True)


@pytest.mark.parametrize("T,K,shared", [(2, 31, True), (5, 31, True), (3, 32, False)])
def test_max_top_k(m, orc, T, K, shared):
    """Slots per token at their cap of 32: 31 routed pairs and the shared
    expert, or 32 routed pairs (2 tokens: 64 slots, one 64-pair grouping
    tile; 5 tokens: 160; 3 tokens: 96)."""
    E, H, I = 40, 512, 256
    check(m, orc, bank_case(95 + T, E, H, I, T, K, shared), E, H, I, 3.0, shared)


@pytest.mark.parametrize("T", [8, 20])
def test_max_experts_shared_with_dropped_ids(m, orc, T):
    """The largest bank the entry point takes (1023 routed experts and the
    shared one, expert id 1023) with dropped pairs, 40 and 100 pairs."""
    E, H, I, K = 1023, 64, 32, 4
    c = bank_case(90 + T, E, H, I, T, K, True)
    c["ids"][0, 0] = -1
    c["ids"][1, 2] = E
    c["ids"][T - 1, 1] = -7
    check(m, orc, c, E, H, I, 1.0, True)


def test_prefill_shape_hot_experts(m, orc, prefill_case):
    """The 256-expert prefill layer at full size with a shared expert and
    limit 10: h of every pair of the three most-routed experts of the
    augmented routing (the shared expert, on all 512 tokens, and the two
    hottest routed ones: every 64-token work item and position), down +
    combine on 32+ tokens (first and last token of each of those items, and
    random ones), end to end on 8 of them."""
    from tests.test_gpu_moe import hot_expert_sample
    cfg = inputs.WORKLOADS[5]
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
    rng = inputs.rng_for(55)
    sh = [inputs.draw_weights(rng, I, H, cfg["scale_lo"], cfg["scale_hi"]),
          inputs.draw_weights(rng, I, H, cfg["scale_lo"], cfg["scale_hi"]),
          inputs.draw_weights(rng, H, I, cfg["scale_lo"], cfg["scale_hi"])]
    c = dict(prefill_case)
    for k, s in zip(("gate", "up", "down"), sh):
        c[k] = np.concatenate([c[k], s])
    ids_a, _, Ea = orc.v41_routing(c["ids"], c["w"], E, True)
    hot, counts, pairs, toks = hot_expert_sample(ids_a, Ea)
    assert hot[0] == E and counts.min() > 64 and len(toks) >= 32
    check(m, orc, c, E, H, I, 10.0, True, tokens=toks, pairs=pairs,
          e2e_tokens=toks[::max(1, len(toks) // 8)], dense=True)


def test_token_alone_equals_batch_bitwise(m):
    E, H, I, T, K = 5, 1024, 512, 80, 2
    c = bank_case(88, E, H, I, T, K, True)
    d = {k: dev(v) for k, v in c.items()}
    ob = host(run(m, d, E, H, I, 3.0, True))
    for t in (0, 41, 79):
        dt = dict(d)
        dt["x"], dt["ids"], dt["w"] = d["x"][t:t + 1], d["ids"][t:t + 1], d["w"][t:t + 1]
        o1 = host(run(m, dt, E, H, I, 3.0, True))
        assert np.array_equal(o1[0], ob[t]), t
