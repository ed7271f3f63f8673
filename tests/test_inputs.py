"""The seeded generators: determinism, shapes, ranges and routing validity."""
import numpy as np

from gemm_mxfp4_dequant_amd import inputs


def test_gemm_case_is_deterministic_and_in_range():
    w1, x1 = inputs.gemm_case(2, 64, 256, 3, 118, 132)
    w2, x2 = inputs.gemm_case(2, 64, 256, 3, 118, 132)
    assert np.array_equal(w1, w2) and np.array_equal(x1, x2)
    assert w1.size == inputs.tensor_nbytes(64, 256) == 64 * 256 * 17 // 32
    sc = w1[64 * 128:]
    assert sc.min() >= 118 and sc.max() <= 132
    assert set(np.unique(sc)) == set(range(118, 133))  # inclusive range
    assert x1.dtype == np.float32 and x1.shape == (3, 256)


def test_code_nibbles_are_uniform():
    w, _ = inputs.gemm_case(3, 512, 512, 1)
    cb = w[: 512 * 256]
    nib = np.concatenate([cb & 15, cb >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16 and counts.max() < 1.1 * nib.size / 16


def test_softmax_routing():
    c = inputs.moe_case(4, 8, 64, 32, 16, 3)
    ids, w = c["ids"], c["w"]
    assert ids.shape == (16, 3) and ids.min() >= 0 and ids.max() < 8
    assert all(len(set(r)) == 3 for r in ids)
    np.testing.assert_allclose(w.sum(1), 1, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # ordered by logit, so by weight


def test_zipf_routing_is_skewed():
    rng = inputs.rng_for(5)
    ids, w = inputs.route_zipf(rng, 512, 256, 8, 1.1)
    assert all(len(set(r)) == 8 for r in ids)
    counts = np.bincount(ids.reshape(-1), minlength=256)
    assert counts.sum() == 4096
    assert counts.max() > 200            # a hot head
    assert (counts <= 8).sum() > 100     # a long cold tail
    np.testing.assert_allclose(w.sum(1), 1, rtol=1e-6)


def test_bf16_draw_is_rounded_fp32():
    rng = inputs.rng_for(6)
    b = inputs.draw_bf16(rng, (4, 64))
    assert b.dtype == np.uint16
    f = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(f))
