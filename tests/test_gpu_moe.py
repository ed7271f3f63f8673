"""GPU parity of the routed expert bank against the oracle.

* grouping (moe_route_group): bit-exact offsets / pair order / slots;
* stage isolation (moe_experts_mxfp4_stages, after the gs_in / gs_out hooks
  of "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs", run_stages):
    h:  |h_gpu - h_or| <= 1e-4 (|silu'(g)| |u| mag_g + |silu(g)| mag_u)
                          + 4 ulp_f32(h)  [+ 1 ulp_bf16(h) when h is bf16]
    down + combine fed with h_gpu:
        |out_gpu - out_or| <= 1e-4 sum_k |w_k| mag_y + 1 ulp_bf16(out_or)
* end to end: nrmse < 1e-3 and cosine > 0.9999 against the oracle's bf16
  output (both sides rounded to bf16; against the unrounded fp64 value the
  bf16 rounding alone is ~1.1e-3 rms);
* invariants: reruns are bitwise equal; out-of-range ids drop pairs.
Workloads: small banks (ragged sizes, scales in the SwiGLU's curved region),
the 64-expert decode layer at full size (every output), and the 256-expert
prefill layer at full size (h of every pair of the three most-routed
experts, down + combine on 32+ tokens).
"""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import assert_within, bf16_to_f64, dev, host, ulp_bf16, ulp_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def upload(c):
    return {k: dev(v) for k, v in c.items()}


def silu_d(g):
    s = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    return s * (1.0 + g * (1.0 - s))


def silu(g):
    return g / (1.0 + np.exp(-np.clip(g, -700, 700)))


def gpu_stages(m, d, E, H, I, xbf):
    """h (slot order) from the stages entry, and the grouping."""
    T, K = d["ids"].shape
    offs, pos, slot = m.moe_route_group(d["ids"], E)
    h = torch.empty((T * K, I), dtype=torch.bfloat16 if xbf else torch.float32, device="cuda")
    m.moe_experts_mxfp4_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"],
                               out=None, h_out=h)
    torch.cuda.synchronize()
    return host(h), host(offs), host(pos), host(slot)


def check_case(m, orc, c, E, H, I, xbf, sample_pairs=None, e2e=True, tokens=None,
               e2e_tokens=None, dense=False):
    """Stage-isolated checks of one bank: h for the pairs ``sample_pairs``
    (all pairs if None), down + combine for ``tokens`` (default: the tokens
    of the checked pairs), end to end for ``e2e_tokens`` (default: the same
    tokens).  ``dense`` computes the oracle's gate/up in its dense form (one
    decode per expert; for many pairs on few experts)."""
    T, K = c["ids"].shape
    P = T * K
    d = upload(c)
    h_gpu, offs, pos, slot = gpu_stages(m, d, E, H, I, xbf)
    # grouping is exact
    counts, offs_o, pos_o, slot_o = orc.group(c["ids"], E)
    assert np.array_equal(offs, offs_o)
    assert np.array_equal(slot, slot_o)
    n_valid = int(offs_o[-1])
    assert np.array_equal(pos[:n_valid], pos_o)

    ids_s = c["ids"].copy().reshape(-1)
    if sample_pairs is not None:
        keep = np.zeros(P, bool)
        keep[sample_pairs] = True
        ids_s[~keep] = -1
    ids_s = ids_s.reshape(T, K)
    gate_up = orc.moe_gate_up_dense if dense else orc.moe_gate_up
    st = gate_up(c["gate"], c["up"], E, H, I, c["x"], ids_s, xbf)
    flat = ids_s.reshape(-1)
    valid = np.where((flat >= 0) & (flat < E))[0]
    hp = h_gpu[slot[valid]]
    hp = bf16_to_f64(hp) if xbf else hp.astype(np.float64)
    g, u = st["g"][valid], st["u"][valid]
    tol_extra = 4 * ulp_f32(st["h"][valid]) + (ulp_bf16(st["h"][valid]) if xbf else 0)
    mag_h = np.abs(silu_d(g)) * np.abs(u) * st["mag_g"][valid] + np.abs(silu(g)) * st["mag_u"][valid]
    assert_within(hp, st["h"][valid], mag_h, extra=tol_extra, what="h")

    # down + combine fed with the device h
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    h_in = dev(h_gpu)
    m.moe_experts_mxfp4_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"],
                               out=out, h_in=h_in)
    out_g = bf16_to_f64(host(out))
    h_pair = np.zeros((P, I))
    vv = np.where(slot >= 0)[0]
    h_pair[vv] = (bf16_to_f64(h_gpu[slot[vv]]) if xbf else h_gpu[slot[vv]].astype(np.float64))
    if tokens is None:
        tok = np.unique(valid // K) if sample_pairs is not None else np.arange(T)
    else:
        tok = np.asarray(tokens)
    ids_t = np.full_like(c["ids"], -1)
    ids_t[tok] = c["ids"][tok]
    y, mag_y = orc.moe_down(c["down"], E, H, I, h_pair, ids_t)
    o, mag_o = orc.moe_combine(y, mag_y, c["w"], ids_t, E)
    assert_within(out_g[tok], o[tok], mag_o[tok], extra=ulp_bf16(o[tok]), what="down+combine")

    if e2e:
        out2 = m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"])
        out2 = bf16_to_f64(host(out2))
        te = tok if e2e_tokens is None else np.asarray(e2e_tokens)
        ids_e = np.full_like(c["ids"], -1)
        ids_e[te] = c["ids"][te]
        # both sides rounded to bf16 (the oracle once, from fp64)
        ref = orc.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], ids_e, c["w"], xbf)
        ref = bf16_to_f64(ref["out_bf16"])[te]
        got = out2[te]
        nrmse = np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
        cos = float((got * ref).sum() / np.sqrt((got * got).sum() * (ref * ref).sum()))
        assert nrmse < 1e-3 and cos > 0.9999, (nrmse, cos)
        return out2


def hot_expert_sample(ids, n_experts, n_hot=3, tpi=64, n_tokens=32, seed=0):
    """Pairs and tokens for a full-size check of a skewed routing: every pair
    (slot) of the ``n_hot`` most-routed experts, so every work item of up to
    ``tpi`` tokens and every position in those items is checked; and at
    least ``n_tokens`` tokens: the first and last token of each such item,
    filled up with seeded random tokens."""
    T, K = ids.shape
    flat = ids.reshape(-1)
    cnt = np.bincount(flat[(flat >= 0) & (flat < n_experts)], minlength=n_experts)
    hot = np.argsort(-cnt, kind="stable")[:n_hot]
    pairs = np.where(np.isin(flat, hot))[0]
    toks = set()
    for e in hot:
        pe = np.where(flat == e)[0]          # the expert's slots, in pair order
        for i0 in range(0, pe.size, tpi):
            item = pe[i0:i0 + tpi]
            toks.update((int(item[0] // K), int(item[-1] // K)))
    rng = np.random.default_rng(seed)
    while len(toks) < n_tokens:
        toks.add(int(rng.integers(T)))
    return hot, cnt[hot], pairs, np.array(sorted(toks))


@pytest.mark.parametrize("xd", ["f32", "bf16"])
@pytest.mark.parametrize("E,H,I,T,K", [(5, 64, 96, 4, 2), (8, 512, 256, 9, 3), (16, 1024, 512, 20, 4),
                                       (3, 96, 160, 1, 3), (33, 2048, 1024, 6, 6),
                                       (4, 512, 1024, 40, 2), (6, 1024, 512, 90, 3),
                                       (40, 512, 512, 16, 4), (40, 512, 512, 13, 5),
                                       (64, 512, 256, 2, 32), (40, 512, 256, 6, 32)])
def test_small_banks(m, orc, xd, E, H, I, T, K):
    # (40, 512, 512, 16, 4) / (40, 512, 512, 13, 5): 64 / 65 pairs, one and
    # two 64-pair tiles of the grouping
    c = inputs.moe_case(E * 100 + T, E, H, I, T, K, xd, "softmax", scale_lo=100, scale_hi=114)
    check_case(m, orc, c, E, H, I, xd == "bf16")


def test_saturated_scales(m, orc):
    c = inputs.moe_case(41, 8, 512, 256, 6, 2, "f32", "softmax", scale_lo=118, scale_hi=132)
    check_case(m, orc, c, 8, 512, 256, False)


def test_dropped_ids(m, orc):
    c = inputs.moe_case(42, 8, 512, 256, 5, 3, "f32", "softmax", scale_lo=100, scale_hi=114)
    c["ids"] = c["ids"].copy()
    c["ids"][1, 2] = -1
    c["ids"][3, 0] = 99
    check_case(m, orc, c, 8, 512, 256, False)


def test_zipf_many_tokens(m, orc):
    """A hot expert with more tokens than one work item holds."""
    rng = inputs.rng_for(43)
    E, H, I, T, K = 16, 512, 256, 200, 4
    c = inputs.moe_case(43, E, H, I, T, K, "bf16", "zipf", scale_lo=100, scale_hi=114)
    assert np.bincount(c["ids"].reshape(-1), minlength=E).max() > 40
    check_case(m, orc, c, E, H, I, True)
    assert rng is not None


def test_row_walk_partial_last_workgroup(m, orc):
    """Gate/up rows 2080 = 130 blocks of 16, walked eight per workgroup (64
    pairs on 64 experts, items of two tokens, the decode layer's kernel):
    each item's last workgroup walks two blocks, and the double-buffered
    reduction alternates within a workgroup; the down product takes 2080
    columns (the generic kernel)."""
    E, H, I, T, K = 64, 4096, 2080, 8, 8
    c = inputs.moe_case(47, E, H, I, T, K, "f32", "softmax", scale_lo=100, scale_hi=114)
    check_case(m, orc, c, E, H, I, False)


def test_workload4_decode_full(m, orc):
    c = inputs.workload_case(4)
    cfg = inputs.WORKLOADS[4]
    check_case(m, orc, c, cfg["n_experts"], cfg["hidden"], cfg["inter"], False)


def test_workload5_prefill_hot_experts(m, orc, prefill_case):
    """The 256-expert prefill layer at full size: h of every pair of the three
    most-routed experts (441, 321 and 236 pairs in this draw: every 64-token
    work item and every position in it), down + combine on 32+ tokens (the
    first and last token of each of those items, and random ones), end to
    end on 8 of them."""
    cfg = inputs.WORKLOADS[5]
    c = prefill_case
    hot, counts, pairs, toks = hot_expert_sample(c["ids"], cfg["n_experts"])
    assert counts.min() > 64 and len(toks) >= 32
    check_case(m, orc, c, cfg["n_experts"], cfg["hidden"], cfg["inter"], True,
               sample_pairs=pairs, tokens=toks, e2e_tokens=toks[::max(1, len(toks) // 8)],
               dense=True)


@pytest.mark.parametrize("xd", ["f32", "bf16"])
def test_tiled_bank_with_few_pair_experts(m, orc, xd):
    """Routing for the tiled path (160 tokens x 3 on 24 experts) with three
    hot experts (~140 pairs each: three 64-token items), twenty experts with
    1, 2, 3 or 4 pairs (their down products one item each on the skinny
    kernel, their gate/up items after the others' in the tiled kernel), one
    with 5 (just past that cut: tiled throughout) and two dropped pairs;
    every pair and token is checked."""
    E, H, I, T, K = 24, 1024, 512, 160, 3
    c = inputs.moe_case(48, E, H, I, T, K, xd, "softmax", scale_lo=100, scale_hi=114)
    ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    cold = [e for e in range(3, 23) for _ in range(1 + (e - 3) % 4)] + [23] * 5
    toks = np.random.default_rng(48).choice(T, len(cold), replace=False)
    for t, e in zip(toks, cold):
        ids[t, t % K] = e            # at most one such expert per token
    rest = np.setdiff1d(np.arange(T), toks)
    ids[rest[0], 1] = -1
    ids[rest[1], 2] = E + 5
    c["ids"] = ids
    cnt = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
    assert cnt[:3].min() > 128 and sorted(set(cnt[3:23])) == [1, 2, 3, 4] and cnt[23] == 5
    check_case(m, orc, c, E, H, I, xd == "bf16")


def test_rerun_bitwise(m):
    E, H, I, T, K = 16, 1024, 512, 12, 4
    c = inputs.moe_case(44, E, H, I, T, K, "f32", "softmax", scale_lo=100, scale_hi=114)
    d = upload(c)
    o1 = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"]))
    o2 = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"]))
    assert np.array_equal(o1, o2)


def test_group_large(m, orc):
    """All three grouping paths: one-wave tile ranking (up to 8 tiles of 64
    pairs), 16-wave tile ranking (up to 128 tiles, histogram within 128 KB
    of LDS) and chunked counting (beyond, up to the 2^25-pair cap); 1024
    experts; ids outside [0, E) in a few cases."""
    rng = np.random.default_rng(45)
    # (the last two: the largest routing the entry points take, 2^20 tokens
    # x top 32 = 33.5 M pairs on 1024 experts, and 2^20 x 8 with dropped ids)
    for (T, K, E, bad) in [(512, 8, 256, 0), (3000, 4, 1024, 0), (1, 1, 1, 0), (7, 32, 40, 0),
                           (1024, 8, 64, 0), (1024, 8, 512, 0), (20, 4, 1024, 0),
                           (100, 6, 50, 9), (1100, 8, 300, 40), (64, 8, 1024, 5),
                           (8, 6, 64, 0), (60, 8, 7, 3), (1 << 20, 32, 1024, 0),
                           (1 << 20, 8, 256, 1000)]:
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
        if bad:
            flat = ids.reshape(-1)
            where = rng.choice(flat.size, bad, replace=False)
            flat[where[: bad // 2]] = -1
            flat[where[bad // 2:]] = E + 3
        offs, pos, slot = m.moe_route_group(dev(ids), E)
        counts, offs_o, pos_o, slot_o = orc.group(ids, E)
        nv = int(offs_o[E])  # pairs with a valid expert; slots past them stay unwritten
        hp = host(pos)
        assert np.array_equal(host(offs), offs_o)
        assert np.array_equal(hp[:nv], pos_o[:nv])
        assert np.all(hp[nv:] == -1)
        assert np.array_equal(host(slot), slot_o)


@pytest.mark.parametrize("xd", ["f32", "bf16"])
@pytest.mark.parametrize("E,H,I,T,K", [(6, 1024, 512, 96, 2), (64, 512, 256, 20, 4)])
def test_token_alone_equals_batch_bitwise(m, xd, E, H, I, T, K):
    """A token's output is the same bits whether the bank runs it in a batch
    or alone: one summation order.  Batches: 96 tokens on 6 experts (tiled
    kernels, items of many tokens) and 20 tokens on 64 experts (80 pairs,
    skinny kernels, items of two tokens)."""
    c = inputs.moe_case(46, E, H, I, T, K, xd, "softmax", scale_lo=100, scale_hi=114)
    d = upload(c)
    ob = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"]))
    for t in (0, 17, T - 1):
        o1 = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"][t:t + 1],
                                      d["ids"][t:t + 1], d["w"][t:t + 1]))
        assert np.array_equal(o1[0], ob[t]), t


@pytest.mark.parametrize("T,K,E,xdt,drop", [(8, 6, 64, "f32", False), (8, 8, 64, "f32", True),
                                            (1, 4, 16, "bf16", False), (16, 4, 40, "f32", True),
                                            (13, 5, 1024, "f32", False)])
def test_fused_grouping_equals_grouping_kernel(m, T, K, E, xdt, drop):
    """Routing of at most 64 pairs is grouped inside the gate/up kernel (each
    workgroup ranks the pairs itself; workgroup 0 writes the tables for down
    and combine); the staged entry point, asked for h, runs the grouping
    kernel instead.  Both must give the same output bit for bit, including
    dropped pairs, a single token, ragged pair counts (13 x 5 = 65 pairs
    takes the grouping kernel on both sides) and a 1024-expert bank."""
    H, I = 512, 64
    c = inputs.moe_case(900 + T * K + E, E, H, I, T, K, xdt, "softmax", scale_lo=110,
                        scale_hi=124)
    ids = c["ids"].copy().reshape(-1)
    if drop:
        ids[::5] = -1
        ids[3::7] = E + 2
    c["ids"] = ids.reshape(T, K).astype(np.int32)
    d = upload(c)
    fused = m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"], d["w"])
    h = torch.empty((T * K, I), dtype=torch.bfloat16 if xdt == "bf16" else torch.float32,
                    device="cuda")
    staged, _ = m.moe_experts_mxfp4_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"],
                                           d["ids"], d["w"], out=torch.empty_like(fused), h_out=h)
    torch.cuda.synchronize()
    a, b = host(fused), host(staged)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    # and a rerun of the fused path (its tables rewritten in the same workspace)
    again = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                     d["w"]))
    assert np.array_equal(a.view(np.uint16), again.view(np.uint16))


@pytest.mark.parametrize("shared", [False, True])
def test_fused_grouping_v41(m, shared):
    """The V4.1 bank on decode-sized routing: the fused grouping's route
    weights (read through its own pair table) and the shared expert's
    augmented routing give the staged (grouping-kernel) result bit for bit."""
    E, H, I, T, K = 32, 1024, 512, 6, 7
    c = inputs.moe_case(77 + int(shared), E + int(shared), H, I, T, K, "bf16", "softmax",
                        scale_lo=110, scale_hi=125)
    ids = c["ids"].copy()
    ids[ids >= E] = ids[ids >= E] % E
    c["ids"] = ids.astype(np.int32)
    d = upload(c)
    fused = m.moe_experts_mxfp4_v41(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                    d["w"], swiglu_limit=7.0, has_shared=shared)
    h = torch.empty((T * (K + int(shared)), I), dtype=torch.bfloat16, device="cuda")
    staged, _ = m.moe_experts_mxfp4_v41_stages(d["gate"], d["up"], d["down"], E, H, I, d["x"],
                                               d["ids"], d["w"], swiglu_limit=7.0,
                                               has_shared=shared, out=torch.empty_like(fused),
                                               h_out=h)
    torch.cuda.synchronize()
    assert np.array_equal(host(fused).view(np.uint16), host(staged).view(np.uint16))


@pytest.mark.parametrize("T,K,E,xdt", [
    (8, 6, 64, "f32"),     # at most 64 pairs: grouping inside the gate/up kernel
    (24, 4, 16, "bf16"),   # grouping kernel, skinny kernels
    (160, 3, 24, "bf16"),  # tiled kernels
])
def test_every_pair_dropped(m, T, K, E, xdt):
    """The method's degenerate routing: every pair dropped (id -1 or
    >= n_experts), so there are no work items and every output is an empty
    weighted sum, +0 in every position (the oracle's combine of no slots).
    The workspace first serves a call with real routing, so the empty call
    must replace that call's item list and slot tables, not reuse them; a
    real call after it gives the first call's bits again.  Plain bank, FP4 x
    FP8 bank and (bf16) V4.1 bank without a shared expert."""
    H = I = 512
    c = inputs.moe_case(4242 + T, E, H, I, T, K, xdt, "softmax", scale_lo=110, scale_hi=124)
    d = upload(c)
    dropped = dev(np.where(np.arange(T * K).reshape(T, K) % 2 == 0, -1, E + 3).astype(np.int32))
    banks = [("plain", m.moe_experts_mxfp4,
              m.moe_experts_mxfp4_workspace_size(T, K, E, H, I, d["x"].dtype)),
             ("a8", m.moe_experts_mxfp4_a8, m.moe_experts_mxfp4_a8_workspace_size(T, K, E, H, I))]
    if xdt == "bf16":
        banks.append(("v41", lambda *a, **k: m.moe_experts_mxfp4_v41(*a, swiglu_limit=7.0, **k),
                      m.moe_experts_mxfp4_v41_workspace_size(T, K, E, H, I, False)))
    for name, fn, need in banks:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        args = (d["gate"], d["up"], d["down"], E, H, I, d["x"])
        real = host(fn(*args, d["ids"], d["w"], workspace=ws))
        empty = host(fn(*args, dropped, d["w"], workspace=ws))
        again = host(fn(*args, d["ids"], d["w"], workspace=ws))
        torch.cuda.synchronize()
        assert real.view(np.uint16).any(), name
        assert not empty.view(np.uint16).any(), (name, np.count_nonzero(empty.view(np.uint16)))
        assert np.array_equal(real.view(np.uint16), again.view(np.uint16)), name


def test_bank_at_token_cap(m, orc):
    """The largest token count the entry points take (MXFP4_MAX_TOKENS = 2^20
    tokens, top 8 of 64 experts: 8.4 M pairs, chunked grouping, skinny
    kernels) at the narrowest widths (hidden = inter = 32): the grouping
    exact, h of 300 sampled pairs (the first and last among them), down +
    combine and end to end for their tokens."""
    E, H, I, T, K = 64, 32, 32, 1 << 20, 8
    c = inputs.moe_case(2020, E, H, I, T, K, "f32", "softmax", scale_lo=110, scale_hi=124)
    rng = np.random.default_rng(7)
    pairs = np.unique(np.concatenate([[0, 1, T * K - 1], rng.integers(0, T * K, 300)]))
    check_case(m, orc, c, E, H, I, False, sample_pairs=pairs)
