"""Pins for the oracle's router (softmax over gating logits, top-k by logit,
renormalised weights; the routing the 64-expert decode workload states).

Each pin checks the oracle against something other than its own code:
repeated arg-max by hand-written scans, permutations of tiny rows, the
two-expert closed form (a logistic function), exact invariants (a shift of
every logit, uniform rows, top-1, top-E), and the workload generator's own
routing of the same draw."""
import itertools
import math

import numpy as np

from gemm_mxfp4_dequant_amd import inputs


def scan_rank(row, k):
    """k rounds of 'take the largest remaining, lowest index on a tie',
    NaN only when no number remains (plain scans, no sorting)."""
    taken = [False] * len(row)
    out = []
    for _ in range(k):
        best = -1
        for e, v in enumerate(row):
            if taken[e]:
                continue
            if best < 0:
                best = e
                continue
            b = row[best]
            if math.isnan(b) and not math.isnan(v):
                best = e
            elif not math.isnan(v) and v > b:
                best = e
        taken[best] = True
        out.append(best)
    return out


def test_rank_order_matches_scans(orc):
    rng = np.random.default_rng(7)
    for E, K in [(1, 1), (5, 2), (64, 6), (65, 7), (256, 8), (1024, 32)]:
        L = rng.standard_normal((6, E)).astype(np.float32)
        ids, _ = orc.route_topk(L, K)
        for t in range(6):
            assert list(ids[t]) == scan_rank([float(v) for v in L[t]], K)


def test_ties_zeros_and_nan_rank(orc):
    """Every ordering of a tiny row with ties, +-0 and NaN ranks as the scans
    do; all-equal rows rank 0, 1, 2, ..."""
    base = [1.0, 1.0, 0.0, -0.0, float("nan"), -math.inf, 2.0]
    for perm in itertools.islice(itertools.permutations(range(7)), 0, 5040, 7):
        row = [base[i] for i in perm]
        ids, _ = orc.route_topk(np.array([row]), 6)
        assert list(ids[0]) == scan_rank(row, 6), row
    ids, w = orc.route_topk(np.full((3, 40), 0.25), 16)
    assert (ids == np.arange(16)).all()
    assert np.allclose(w, 1.0 / 16, rtol=0, atol=1e-16)


def test_two_experts_closed_form(orc):
    """E = K = 2: w_0 = 1 / (1 + e^(l_1 - l_0)) with l_0 the larger logit."""
    rng = np.random.default_rng(8)
    L = rng.normal(0, 3, (200, 2))
    ids, w = orc.route_topk(L, 2)
    hi = L.max(axis=1)
    lo = L.min(axis=1)
    want = 1.0 / (1.0 + np.exp(lo - hi))
    assert np.array_equal(ids[:, 0], np.argmax(L, axis=1))
    assert np.allclose(w[:, 0], want, rtol=1e-15, atol=0)
    assert np.allclose(w[:, 1], 1.0 - want, rtol=1e-13, atol=1e-16)


def test_invariants(orc):
    """Shifting every logit changes nothing; weights sum to 1, are positive
    and descend with rank; top-1 weighs 1; top-E keeps every expert."""
    rng = np.random.default_rng(9)
    L = rng.standard_normal((50, 64))
    ids, w = orc.route_topk(L, 8)
    ids2, w2 = orc.route_topk(L + 37.5, 8)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w, w2, rtol=1e-12, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (w > 0).all() and (np.diff(w, axis=1) <= 0).all()
    ids1, w1 = orc.route_topk(L, 1)
    assert (w1 == 1.0).all() and np.array_equal(ids1[:, 0], np.argmax(L, axis=1))
    idsE, wE = orc.route_topk(L[:, :16], 16)
    p = np.exp(L[:, :16] - L[:, :16].max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(wE, np.take_along_axis(p, idsE, axis=1), rtol=1e-14, atol=0)


def test_minus_inf_gets_zero_weight(orc):
    L = np.array([[0.5, -np.inf, 0.25, -np.inf]])
    ids, w = orc.route_topk(L, 3)
    assert list(ids[0]) == [0, 2, 1]
    assert w[0, 2] == 0.0
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-0.25))) < 1e-15


def test_matches_the_decode_workload_routing(orc):
    """The workload generator routes its own draw (fp32 weights); the oracle
    on the same logits agrees: same ids, weights within fp32 rounding."""
    T, E, K = 8, 64, 6
    ids_g, w_g = inputs.route_softmax(inputs.rng_for(99), T, E, K)
    L = inputs.gating_logits(inputs.rng_for(99), T, E)
    ids, w = orc.route_topk(L, K)
    assert np.array_equal(ids, ids_g)
    assert np.allclose(w, w_g, rtol=2 ** -23, atol=0)
