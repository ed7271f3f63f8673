"""Shared helpers for the GPU parity tests: device upload and the tolerance
rules.

Tolerances (the pass rule for floating point):
  * dense products: |y_gpu - y_oracle| <= 1e-4 * sum|w*x| + 1e-30 per output
    (fp32 accumulation order differs; the floor follows the pages' device
    test in "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs");
  * a NaN output must be NaN on both sides;
  * dequantization: bit-exact.
"""
import numpy as np
import torch

REL = 1e-4
FLOOR = 1e-30


def dev(a, dtype=None):
    """numpy -> torch cuda tensor (uint16 arrays are bf16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_within(got, want, mag, rel=REL, floor=FLOOR, extra=0.0, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    mag = np.asarray(mag, np.float64)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{what}: NaN pattern differs"
    ok = ~nan_w
    err = np.abs(got[ok] - want[ok])
    tol = rel * mag[ok] + floor + (extra[ok] if isinstance(extra, np.ndarray) else extra)
    bad = err > tol
    if bad.any():
        i = np.argmax(err - tol)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                             f"got {got[ok][i]!r} want {want[ok][i]!r} tol {tol[i]!r} "
                             f"(err/mag {err[i] / max(mag[ok][i], 1e-300):.3e})")
    return float((err / np.maximum(mag[ok], 1e-300)).max()) if err.size else 0.0


def ulp_bf16(v):
    """Spacing of bf16 numbers at |v| (normal range)."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def ulp_f32(v):
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 23)


def sync():
    torch.cuda.synchronize()
