"""Seeded synthetic inputs for the MXFP4 path (shared by tests, bench and the
oracle's callers).

This module holds none of the method's arithmetic: it draws random bytes,
activations and routings and lays them out as the operands of the path.  A
weight tensor is drawn directly in its stored form: the code plane as uniform
random bytes (so every nibble is iid uniform over 0..15 and 1/16 of the
weights are -0) followed by the scale plane as uniform integers over an
inclusive range.  No packing or decoding happens here.

Draw order for a seed: weights (per role, per expert: codes then scales),
then activations, then routing.  Generator: numpy PCG64.

Workloads (the five measured shapes):
  1  matvec [256 x 512], scales 120..130, one fp32 row
  2  matvec/GEMM [4096 x 4096], scales 118..132, fp32 rows, b = 1 and 8
  3  GEMM [14336 x 4096], scales 118..132, fp32 rows, b = 1, 2, 4, 8, 16, 32
  4  MoE decode: 64 experts, hidden 4096, inter 2048, 8 tokens, top-6 by
     softmax over N(0,1) logits, renormalised; fp32 in, bf16 out
  5  MoE prefill: 256 experts, hidden 7168, inter 2048, 512 tokens, top-8 with
     Zipf(1.1) expert popularity; bf16 in, bf16 out
The MoE workloads give no scale range; the GEMM range 118..132 is used.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    1: dict(kind="gemm", rows=256, cols=512, scale_lo=120, scale_hi=130, batches=(1,)),
    2: dict(kind="gemm", rows=4096, cols=4096, scale_lo=118, scale_hi=132, batches=(1, 8)),
    3: dict(kind="gemm", rows=14336, cols=4096, scale_lo=118, scale_hi=132,
            batches=(1, 2, 4, 8, 16, 32)),
    4: dict(kind="moe", n_experts=64, hidden=4096, inter=2048, n_tokens=8, top_k=6,
            x_dtype="f32", routing="softmax", scale_lo=118, scale_hi=132),
    5: dict(kind="moe", n_experts=256, hidden=7168, inter=2048, n_tokens=512, top_k=8,
            x_dtype="bf16", routing="zipf", zipf_s=1.1, scale_lo=118, scale_hi=132),
}


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tensor_nbytes(rows: int, cols: int) -> int:
    """Stored size of a rows x cols tensor (codes, then one scale per 32)."""
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    return rows * cols // 2 + rows * (cols // 32)


def draw_weights(rng: np.random.Generator, rows: int, cols: int, scale_lo: int,
                 scale_hi: int, count: int = 1) -> np.ndarray:
    """``count`` consecutive stored tensors (codes then scales each), uint8."""
    code_bytes = rows * cols // 2
    n_scales = rows * (cols // 32)
    out = np.empty(count * (code_bytes + n_scales), np.uint8)
    stride = code_bytes + n_scales
    for i in range(count):
        base = i * stride
        out[base:base + code_bytes] = np.frombuffer(rng.bytes(code_bytes), np.uint8)
        out[base + code_bytes:base + stride] = rng.integers(
            scale_lo, scale_hi + 1, size=n_scales, dtype=np.uint8)
    return out


def draw_f32(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 N(0, 1)."""
    return rng.standard_normal(shape, dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, nearest-even, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 N(0, 1): an fp32 draw rounded to bf16; returned as uint16 bits."""
    return to_bf16_bits(draw_f32(rng, shape))


def gating_logits(rng: np.random.Generator, n_tokens: int, n_experts: int) -> np.ndarray:
    """N(0,1) fp32 gating logits [n_tokens, n_experts]."""
    return rng.standard_normal((n_tokens, n_experts), dtype=np.float32)


def route_softmax(rng: np.random.Generator, n_tokens: int, n_experts: int, top_k: int):
    """The 64-expert decode workload's routing, drawn for its inputs: N(0,1)
    logits, softmax in fp64, top-k by logit (lower index wins a tie),
    weights renormalised over the chosen k and stored as fp32."""
    logits = gating_logits(rng, n_tokens, n_experts).astype(np.float64)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(p, order, axis=1)
    w = (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def route_zipf(rng: np.random.Generator, n_tokens: int, n_experts: int, top_k: int,
               s: float):
    """Zipf(s) expert popularity over a seeded permutation of the experts;
    each token takes the top-k of log p_e + Gumbel(0,1) (sampling without
    replacement with probability proportional to p), and its weights are a
    softmax over the k selected scores, stored as fp32."""
    perm = rng.permutation(n_experts)
    rank = np.empty(n_experts, np.float64)
    rank[perm] = np.arange(1, n_experts + 1, dtype=np.float64)
    logp = -s * np.log(rank)
    logp -= np.log(np.exp(logp).sum())
    scores = logp[None, :] + rng.gumbel(size=(n_tokens, n_experts))
    order = np.argsort(-scores, axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(scores, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w


def gemm_case(seed: int, rows: int, cols: int, b: int, scale_lo=118, scale_hi=132,
              x_dtype="f32"):
    """One weight tensor and b activation rows [b, cols]."""
    rng = rng_for(seed)
    w = draw_weights(rng, rows, cols, scale_lo, scale_hi)
    x = draw_f32(rng, (b, cols)) if x_dtype == "f32" else draw_bf16(rng, (b, cols))
    return w, x


def moe_case(seed: int, n_experts: int, hidden: int, inter: int, n_tokens: int, top_k: int,
             x_dtype="f32", routing="softmax", zipf_s=1.1, scale_lo=118, scale_hi=132):
    """Expert bank (gate, up: [inter x hidden]; down: [hidden x inter], each
    n_experts contiguous tensors), activations [n_tokens, hidden] and the
    routing (ids int32 and weights fp32, [n_tokens, top_k])."""
    rng = rng_for(seed)
    gate = draw_weights(rng, inter, hidden, scale_lo, scale_hi, n_experts)
    up = draw_weights(rng, inter, hidden, scale_lo, scale_hi, n_experts)
    down = draw_weights(rng, hidden, inter, scale_lo, scale_hi, n_experts)
    x = (draw_f32(rng, (n_tokens, hidden)) if x_dtype == "f32"
         else draw_bf16(rng, (n_tokens, hidden)))
    if routing == "softmax":
        ids, w = route_softmax(rng, n_tokens, n_experts, top_k)
    else:
        ids, w = route_zipf(rng, n_tokens, n_experts, top_k, zipf_s)
    return dict(gate=gate, up=up, down=down, x=x, ids=ids, w=w)


def workload_case(n: int, seed: int | None = None, b: int | None = None):
    """Inputs of workload ``n`` (seed defaults to n)."""
    cfg = WORKLOADS[n]
    seed = n if seed is None else seed
    if cfg["kind"] == "gemm":
        bb = b if b is not None else max(cfg["batches"])
        return gemm_case(seed, cfg["rows"], cfg["cols"], bb, cfg["scale_lo"], cfg["scale_hi"])
    return moe_case(seed, cfg["n_experts"], cfg["hidden"], cfg["inter"], cfg["n_tokens"],
                    cfg["top_k"], cfg["x_dtype"], cfg["routing"], cfg.get("zipf_s", 1.1),
                    cfg["scale_lo"], cfg["scale_hi"])


def draw_weights_device(seed: int, rows: int, cols: int, scale_lo: int, scale_hi: int,
                        count: int, device="cuda"):
    """``count`` stored tensors drawn on the device with a seeded torch
    generator (same distributions as ``draw_weights``; used for the large
    rotating pools of the benchmark).  Returns a uint8 tensor [count, bytes]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    code_bytes = rows * cols // 2
    n_scales = rows * (cols // 32)
    out = torch.empty((count, code_bytes + n_scales), dtype=torch.uint8, device=device)
    for i in range(count):
        out[i, :code_bytes] = torch.randint(0, 256, (code_bytes,), generator=g, device=device,
                                            dtype=torch.uint8)
        out[i, code_bytes:] = torch.randint(scale_lo, scale_hi + 1, (n_scales,), generator=g,
                                            device=device, dtype=torch.uint8)
    return out
