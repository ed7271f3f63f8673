"""GPU parity of the device router (moe_route_topk) against the oracle.

* ids: bit-exact (the selection compares the fp32 logits themselves, on
  both sides, so it is an exact integer decision);
* weights: fp32 expf of d_k = l_k - l_0, summed over k slots in fp32, one
  division.  Relative error of w_k is at most
      (|d_k| + max_j |d_j|) 2^-24   (rounding of the fp32 differences)
    + 2 * 2^-23                      (expf, in the term and through the sum)
    + (K - 1) 2^-24 + 2^-24          (the sum, the division)
  so the test allows twice that, relative to the oracle's fp64 weight, plus
  an absolute 1e-37 for terms that underflow fp32;
* the router's output drives the expert bank exactly as host-side ids and
  weights do.
Shapes: the 64-expert decode routing (8 tokens, top 6), the prefill size
(512 x 256, top 8), the limits (1024 experts, top 32), ragged expert counts,
rows with many ties, signed zeros, -inf, NaN and extreme magnitudes.
"""
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


def w_bound(L, ids, w_or):
    K = ids.shape[1]
    Lf = L.astype(np.float64)
    sel = np.take_along_axis(Lf, ids.astype(np.int64), axis=1)
    d = np.abs(sel - sel[:, :1])
    d = np.where(np.isfinite(d), d, 0.0)
    rel = (d + d.max(axis=1, keepdims=True) + 2 * 2 + K) * 2.0 ** -24
    return 2 * rel * np.abs(w_or) + 1e-37


def check(m, orc, L, K):
    ids, w = m.moe_route_topk(dev(np.ascontiguousarray(L, np.float32)), K)
    torch.cuda.synchronize()
    ids, w = host(ids), host(w).astype(np.float64)
    ids_o, w_o = orc.route_topk(L.astype(np.float32), K)
    assert np.array_equal(ids, ids_o)
    err = np.abs(w - w_o)
    tol = w_bound(L.astype(np.float32), ids_o, w_o)
    assert (err <= tol).all(), (err / np.maximum(tol, 1e-300)).max()
    return ids, w


@pytest.mark.parametrize("T,E,K", [(8, 64, 6), (512, 256, 8), (300, 1024, 32), (1, 1, 1),
                                   (5, 65, 7), (7, 1000, 3), (33, 32, 32), (2, 2, 2)])
def test_random_logits(m, orc, T, E, K):
    L = inputs.gating_logits(inputs.rng_for(T * 1000 + E), T, E)
    check(m, orc, L, K)


def test_decode_workload_routing(m, orc):
    """The decode workload's own draw: the device router reproduces the ids
    the workload generator chose, and weights within the bound."""
    T, E, K = 8, 64, 6
    ids_g, w_g = inputs.route_softmax(inputs.rng_for(4), T, E, K)
    L = inputs.gating_logits(inputs.rng_for(4), T, E)
    ids, w = check(m, orc, L, K)
    assert np.array_equal(ids, ids_g)
    assert np.allclose(w, w_g, rtol=2e-6, atol=0)


def test_ties(m, orc):
    """Integer logits in [-2, 2] (many equal values): lower index first."""
    rng = np.random.default_rng(3)
    L = rng.integers(-2, 3, size=(64, 100)).astype(np.float32)
    check(m, orc, L, 16)
    check(m, orc, np.zeros((4, 70), np.float32), 9)


def test_special_values(m, orc):
    """+-0 ties, -inf entries (weight 0 when chosen), NaN entries (ranked
    last: fewer NaN than E - K per row so none is chosen), and logits near
    the fp32 limits."""
    rng = np.random.default_rng(4)
    T, E, K = 40, 96, 8
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[0, :] = 0.0
    L[0, ::3] = -0.0
    L[1, :90] = -np.inf
    L[2, rng.choice(E, 30, replace=False)] = np.nan
    L[3, :] = rng.choice([3e38, -3e38, 1e30, -1e-30], size=E).astype(np.float32)
    L[4, :] = np.float32(1e-44)  # subnormal ties
    L[5, 17] = np.inf             # one +inf: chosen first, weights NaN on both sides
    ids, w = m.moe_route_topk(dev(L), K)
    ids, w = host(ids), host(w).astype(np.float64)
    ids_o, w_o = orc.route_topk(L, K)
    assert np.array_equal(ids, ids_o)
    assert ids[5, 0] == 17 and np.isnan(w[5]).all()
    keep = np.ones(T, bool)
    keep[5] = False
    err = np.abs(w[keep] - w_o[keep])
    assert (err <= w_bound(L[keep], ids_o[keep], w_o[keep])).all()
    # row 1: six finite logits (experts 90..95) rank first; the two -inf picks weigh 0
    assert (ids[1, :6] >= 90).all() and (w[1, 6:] == 0).all() and (w[1, :6] > 0).all()


def test_rerun_bitwise(m):
    L = dev(inputs.gating_logits(inputs.rng_for(5), 257, 300))
    a = [host(t) for t in m.moe_route_topk(L, 11)]
    b = [host(t) for t in m.moe_route_topk(L, 11)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32),
                                                          b[1].view(np.uint32))


def test_router_drives_the_bank(m):
    """Device routing -> expert bank equals the bank fed with the same ids
    and weights copied through the host: the router's output is the bank's
    input format."""
    E, H, I, T, K = 16, 512, 256, 24, 4
    c = inputs.moe_case(71, E, H, I, T, K, "f32", "softmax", scale_lo=100, scale_hi=114)
    d = {k: dev(v) for k, v in c.items()}
    L = dev(inputs.gating_logits(inputs.rng_for(72), T, E))
    ids, w = m.moe_route_topk(L, K)
    o1 = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], ids, w))
    ids_h, w_h = dev(host(ids)), dev(host(w))
    o2 = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], ids_h, w_h))
    assert np.array_equal(o1, o2)
