"""CPU oracle for the MXFP4 dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it imports nothing from the HIP side.

The arithmetic lives in ``mxfp4_oracle.c`` (plain C, fp64, one term at a time);
this module builds it with gcc and marshals numpy arrays.  Inputs given as
fp32 or bf16 are widened to fp64 exactly before the C code sees them.

Parity status of each function is stated in its docstring ("pinned by ...").
Nothing in the oracle is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile ``mxfp4_oracle.c`` into ``liboracle.so`` with gcc (always)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_e2m1.restype = ctypes.c_double
    lib.orc_e2m1.argtypes = [ctypes.c_int]
    lib.orc_e8m0.restype = ctypes.c_double
    lib.orc_e8m0.argtypes = [ctypes.c_int]
    lib.orc_nbytes.restype = I64
    lib.orc_nbytes.argtypes = [I64, I64]
    lib.orc_dequant_value_f32.restype = ctypes.c_float
    lib.orc_dequant_value_f32.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.orc_dequant_f32.restype = None
    lib.orc_dequant_f32.argtypes = [P, I64, I64, P]
    lib.orc_dequant_bf16.restype = None
    lib.orc_dequant_bf16.argtypes = [P, I64, I64, P]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne.argtypes = [ctypes.c_double]
    lib.orc_bf16_rne_n.restype = None
    lib.orc_bf16_rne_n.argtypes = [P, I64, P]
    lib.orc_e4m3.restype = ctypes.c_double
    lib.orc_e4m3.argtypes = [ctypes.c_int]
    lib.orc_e4m3_rne.restype = ctypes.c_int
    lib.orc_e4m3_rne.argtypes = [ctypes.c_double]
    lib.orc_mxfp8_quantize.restype = None
    lib.orc_mxfp8_quantize.argtypes = [P, I64, I64, P, P]
    lib.orc_gemm.restype = None
    lib.orc_gemm.argtypes = [P, I64, I64, P, I64, P, P, ctypes.c_int]
    lib.orc_gemm_rows.restype = None
    lib.orc_gemm_rows.argtypes = [P, I64, I64, P, I64, P, I64, P, P, ctypes.c_int]
    lib.orc_group.restype = None
    lib.orc_group.argtypes = [P, I64, I64, P, P, P, P]
    lib.orc_moe_gate_up.restype = None
    lib.orc_moe_gate_up.argtypes = [P, P, I64, I64, P, P, I64, I64, ctypes.c_int,
                                    P, P, P, P, P, ctypes.c_int]
    lib.orc_moe_down.restype = None
    lib.orc_moe_down.argtypes = [P, I64, I64, P, P, I64, I64, P, P, ctypes.c_int]
    lib.orc_moe_v41_act.restype = None
    lib.orc_moe_v41_act.argtypes = [P, P, P, P, I64, I64, ctypes.c_double, P]
    lib.orc_moe_combine.restype = None
    lib.orc_moe_combine.argtypes = [P, P, P, P, I64, I64, I64, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_f64(x) -> np.ndarray:
    """Widen an activation array to fp64 exactly.

    ``x`` is fp32, fp64, or bf16 given as its uint16 bit patterns (numpy has no
    bf16); a bf16 pattern is the top half of the fp32 with the same value.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _as_bytes(w) -> np.ndarray:
    w = np.ascontiguousarray(np.asarray(w), dtype=np.uint8).reshape(-1)
    return w


# --------------------------------------------------------------------------
# Format
# --------------------------------------------------------------------------

def e2m1(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign bit 3).  Pinned by test_oracle_format."""
    return _load().orc_e2m1(int(code))


def e8m0(k: int) -> float:
    """Value of an E8M0 scale byte.  Pinned by test_oracle_format."""
    return _load().orc_e8m0(int(k))


def nbytes(rows: int, cols: int) -> int:
    """Byte size of a rows x cols MXFP4 tensor (-1 if cols % 32 != 0)."""
    return int(_load().orc_nbytes(rows, cols))


def dequant_value_f32(code: int, k: int) -> np.float32:
    """fp32 weight for one (code, scale byte) pair.  Pinned exhaustively."""
    return np.float32(_load().orc_dequant_value_f32(int(code), int(k)))


def dequant_f32(w, rows: int, cols: int) -> np.ndarray:
    """Bit-exact fp32 dequantization, [rows, cols].  Pinned by the format,
    layout and one-hot tests."""
    w = _as_bytes(w)
    assert w.size >= nbytes(rows, cols) >= 0
    out = np.empty((rows, cols), np.float32)
    _load().orc_dequant_f32(_ptr(w), rows, cols, _ptr(out))
    return out


def dequant_bf16(w, rows: int, cols: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of the dequantized weights, [rows, cols]."""
    w = _as_bytes(w)
    assert w.size >= nbytes(rows, cols) >= 0
    out = np.empty((rows, cols), np.uint16)
    _load().orc_dequant_bf16(_ptr(w), rows, cols, _ptr(out))
    return out


def bf16_rne(v: float) -> int:
    """bf16 bit pattern of an fp64 value, nearest-even.  Pinned by
    test_oracle_bf16 (exact rational search and the pages' fp32 rule)."""
    return int(_load().orc_bf16_rne(float(v)))


def bf16_rne_array(a) -> np.ndarray:
    """bf16_rne of every element (flattened), as uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64).reshape(-1))
    out = np.empty(a.size, np.uint16)
    _load().orc_bf16_rne_n(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# MXFP8 activations (the opt-in block-scaled FP4 x FP8 product)
# --------------------------------------------------------------------------

def e4m3(code: int) -> float:
    """Value of an E4M3 code.  Pinned by test_oracle_mx8."""
    return _load().orc_e4m3(int(code))


def e4m3_rne(v: float) -> int:
    """Nearest E4M3 code (ties to even, saturating).  Pinned by
    test_oracle_mx8."""
    return int(_load().orc_e4m3_rne(float(v)))


def mxfp8_quantize(x):
    """MXFP8 quantization of activations [b, cols] (cols % 32 == 0):
    E4M3 codes uint8 [b, cols] and E8M0 scale bytes uint8 [b, cols/32].
    Pinned by test_oracle_mx8."""
    x = _as_f64(x)
    b, cols = x.shape
    assert cols % 32 == 0
    q = np.empty((b, cols), np.uint8)
    s = np.empty((b, cols // 32), np.uint8)
    _load().orc_mxfp8_quantize(_ptr(x), b, cols, _ptr(q), _ptr(s))
    return q, s


def mxfp8_dequantize(q, s) -> np.ndarray:
    """fp64 values of MXFP8 activations: e4m3(q) * 2^(s - 127) (NaN for a
    scale byte of 255)."""
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.uint8)
    tab = np.array([e4m3(c) for c in range(256)], np.float64)
    sc = np.where(s == 255, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127))
    return tab[q] * np.repeat(sc, 32, axis=1)


def gemm_a8(w, rows: int, cols: int, x, threads: int | None = None):
    """The block-scaled FP4 x FP8 product: the exact product (``gemm``) of
    the weights with the MXFP8-quantized activations.  Returns
    (y [b, rows] fp64, mag = sum |w * x_q|)."""
    q, s = mxfp8_quantize(x)
    return gemm(w, rows, cols, mxfp8_dequantize(q, s), threads)


# --------------------------------------------------------------------------
# Dense product
# --------------------------------------------------------------------------

def gemm(w, rows: int, cols: int, x, threads: int | None = None):
    """y[t, r] = sum_c W[r, c] x[t, c] and mag[t, r] = sum_c |W[r, c] x[t, c]|,
    both fp64, shape [b, rows].  ``x`` is [b, cols] (fp32, fp64 or bf16 bits).
    Pinned by closed forms, one-hot placement and exact-rational brute force."""
    w = _as_bytes(w)
    x = _as_f64(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    b = x.shape[0]
    assert x.shape[1] == cols and w.size >= nbytes(rows, cols) >= 0
    y = np.empty((b, rows), np.float64)
    mag = np.empty((b, rows), np.float64)
    _load().orc_gemm(_ptr(w), rows, cols, _ptr(x), b, _ptr(y), _ptr(mag),
                     threads or default_threads())
    return y, mag


def gemm_rows(w, rows: int, cols: int, x, row_list, threads: int | None = None):
    """``gemm`` restricted to the listed rows: returns ([b, n], [b, n])."""
    w = _as_bytes(w)
    x = _as_f64(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    b = x.shape[0]
    rl = np.ascontiguousarray(row_list, dtype=np.int64)
    assert rl.min() >= 0 and rl.max() < rows
    y = np.empty((b, rl.size), np.float64)
    mag = np.empty((b, rl.size), np.float64)
    _load().orc_gemm_rows(_ptr(w), rows, cols, _ptr(x), b, _ptr(rl), rl.size,
                          _ptr(y), _ptr(mag), threads or default_threads())
    return y, mag


# --------------------------------------------------------------------------
# Routed expert bank
# --------------------------------------------------------------------------

def group(topk_ids, n_experts: int):
    """Stable counting sort of pairs by expert.

    Returns (counts[E], offsets[E+1], pair_of_slot[n_valid], slot_of_pair[P]);
    ids outside [0, E) get slot -1.  Pinned by test_oracle_moe against
    Python's stable ``sorted``."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    P = ids.size
    counts = np.empty(max(n_experts, 1), np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    pos = np.full(max(P, 1), -1, np.int32)
    slot = np.empty(max(P, 1), np.int32)
    _load().orc_group(_ptr(ids), P, n_experts, _ptr(counts), _ptr(offsets),
                      _ptr(pos), _ptr(slot))
    n_valid = int(offsets[n_experts])
    return counts[:n_experts], offsets, pos[:n_valid], slot[:P]


def route_topk(logits, top_k: int):
    """Router: for each token, the softmax of its gating logits (fp64), the
    top_k experts by logit, and their probabilities renormalised to sum to 1.

    The pages give no router (their MoE frame takes picks and weights as
    inputs); this is the routing stated for the 64-expert decode workload
    (softmax over the logits, top 6, renormalised), with these readings:
    larger logit first, equal logits lower index first, -0 equal to +0, and
    NaN ranked below every number and given probability 0.  Returns
    (ids int32 [T, K], w fp64 [T, K]).  Pinned by test_oracle_router
    (exhaustive rank order on small rows, two-expert closed form, shift
    invariance, uniform rows)."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float64)
    for t in range(T):
        row = L[t]
        nan = np.isnan(row)
        # rank: numbers by descending value (+0 and -0 compare equal), then
        # NaN; the expert index breaks ties
        order = sorted(range(E), key=lambda e: (bool(nan[e]), 0.0 if nan[e] else -row[e], e))
        chosen = order[:top_k]
        v = np.where(nan, -np.inf, row)
        z = np.exp(v - v.max())
        p = z / z.sum()
        sel = p[chosen]
        ids[t] = chosen
        w[t] = sel / sel.sum()
    return ids, w


def _sanitize_ids(topk_ids, n_experts):
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).copy()
    ids[(ids < 0) | (ids >= n_experts)] = -1
    return ids


def moe_gate_up(gate, up, n_experts, hidden, inter, x, topk_ids, round_h_bf16,
                threads=None):
    """g, u, h = silu(g)*u (fp64; h optionally rounded to bf16) and the
    magnitudes, each [P, inter] with P = n_tokens * top_k in pair order."""
    x = _as_f64(x)
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    P = T * K
    gate = _as_bytes(gate)
    up = _as_bytes(up)
    need = n_experts * nbytes(inter, hidden)
    assert gate.size >= need and up.size >= need and x.shape == (T, hidden)
    out = {k: np.zeros((P, inter), np.float64) for k in ("g", "u", "h", "mag_g", "mag_u")}
    _load().orc_moe_gate_up(_ptr(gate), _ptr(up), hidden, inter, _ptr(x), _ptr(ids), P, K,
                            int(bool(round_h_bf16)), _ptr(out["g"]), _ptr(out["u"]),
                            _ptr(out["h"]), _ptr(out["mag_g"]), _ptr(out["mag_u"]),
                            threads or default_threads())
    return out


def moe_down(down, n_experts, hidden, inter, h, topk_ids, threads=None):
    """y[p] = W_down[e_p] . h[p] and its magnitudes, [P, hidden] fp64."""
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    P = T * K
    h = _as_f64(h)
    down = _as_bytes(down)
    assert h.shape == (P, inter) and down.size >= n_experts * nbytes(hidden, inter)
    y = np.zeros((P, hidden), np.float64)
    mag = np.zeros((P, hidden), np.float64)
    _load().orc_moe_down(_ptr(down), hidden, inter, _ptr(h), _ptr(ids), P, K, _ptr(y),
                         _ptr(mag), threads or default_threads())
    return y, mag


def moe_combine(y, mag_y, topk_w, topk_ids, n_experts):
    """out[t] = sum_k w[t,k] y[t*K+k] in fp64 (slot order), with magnitudes."""
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    hidden = y.shape[1]
    y = np.ascontiguousarray(y, np.float64)
    mag_y = np.ascontiguousarray(mag_y, np.float64)
    w = np.ascontiguousarray(topk_w, np.float64).reshape(T, K)
    out = np.empty((T, hidden), np.float64)
    mag = np.empty((T, hidden), np.float64)
    _load().orc_moe_combine(_ptr(y), _ptr(mag_y), _ptr(w), _ptr(ids), T, K, hidden,
                            _ptr(out), _ptr(mag))
    return out, mag


def moe(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w, round_h_bf16,
        threads=None):
    """The whole expert bank: gate/up -> SwiGLU -> down -> weighted sum.

    Returns a dict with the stage results (pair order) and ``out`` (fp64),
    ``out_bf16`` (bit patterns, rounded once from fp64) and ``mag_out``."""
    st = moe_gate_up(gate, up, n_experts, hidden, inter, x, topk_ids, round_h_bf16, threads)
    y, mag_y = moe_down(down, n_experts, hidden, inter, st["h"], topk_ids, threads)
    out, mag_out = moe_combine(y, mag_y, topk_w, topk_ids, n_experts)
    st.update(y=y, mag_y=mag_y, out=out, mag_out=mag_out, out_bf16=bf16_rne_array(out).reshape(out.shape))
    return st


# --------------------------------------------------------------------------
# Dense form of the expert stages: the method's plain definition written out
# per expert (dequantize the expert's tensors exactly, then dense fp64
# products of the routed rows), with numpy's fp64 matrix product as the
# library step.  Same results as moe_gate_up / moe_down up to fp64 rounding
# (pinned against them in test_oracle_moe), but each expert is decoded once
# instead of once per pair, so full-size layers can be checked pair by pair
# in seconds.  Valid when no weight overflows fp32 (scale bytes up to 252;
# asserted); a scale of 255 gives NaN rows as in the loop form.
# --------------------------------------------------------------------------

def _expert_f64(bank, e, rows, cols):
    nb = nbytes(rows, cols)
    wf = dequant_f32(bank[e * nb:(e + 1) * nb], rows, cols)
    assert not np.isinf(wf).any(), "dense oracle form: a weight overflows fp32"
    return wf.astype(np.float64)


def moe_gate_up_dense(gate, up, n_experts, hidden, inter, x, topk_ids, round_h_bf16):
    """moe_gate_up in dense form (see above): the same dict, [P, inter]
    each, rows of pairs with invalid ids left at 0.  Pinned against
    moe_gate_up in test_oracle_moe."""
    x = _as_f64(x)
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    P = T * K
    gate = _as_bytes(gate)
    up = _as_bytes(up)
    assert x.shape == (T, hidden)
    out = {k: np.zeros((P, inter), np.float64) for k in ("g", "u", "h", "mag_g", "mag_u")}
    flat = ids.reshape(-1)
    for e in np.unique(flat[flat >= 0]):
        pe = np.where(flat == e)[0]
        xe = x[pe // K]
        for name, bank in (("g", gate), ("u", up)):
            W = _expert_f64(bank, int(e), inter, hidden)
            out[name][pe] = xe @ W.T
            out["mag_" + name][pe] = np.abs(xe) @ np.abs(W).T
    g, u = out["g"], out["u"]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    if round_h_bf16:
        h = bf16_bits_to_f64(bf16_rne_array(h)).reshape(h.shape)
    h[flat < 0] = 0.0
    out["h"] = h
    return out


def moe_down_dense(down, n_experts, hidden, inter, h, topk_ids):
    """moe_down in dense form: y[p] = W_down[e_p] . h[p] and its magnitudes,
    [P, hidden] fp64 (zeros for pairs with invalid ids).  Pinned against
    moe_down in test_oracle_moe."""
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    P = T * K
    h = _as_f64(h)
    down = _as_bytes(down)
    assert h.shape == (P, inter)
    y = np.zeros((P, hidden), np.float64)
    mag = np.zeros((P, hidden), np.float64)
    flat = ids.reshape(-1)
    for e in np.unique(flat[flat >= 0]):
        pe = np.where(flat == e)[0]
        W = _expert_f64(down, int(e), hidden, inter)
        y[pe] = h[pe] @ W.T
        mag[pe] = np.abs(h[pe]) @ np.abs(W).T
    return y, mag


def moe_v41_act(g, u, topk_w, topk_ids, n_experts, swiglu_limit):
    """V4.1 activation of every pair: h = bf16(w * silu(min(bf16 g, lim)) *
    clamp(bf16 u, -lim, lim)) (no clamping when lim <= 0); [P, inter] fp64
    holding bf16 values, pairs with invalid ids left at 0."""
    ids = _sanitize_ids(topk_ids, n_experts)
    T, K = ids.shape
    P = T * K
    g = np.ascontiguousarray(g, np.float64)
    u = np.ascontiguousarray(u, np.float64)
    assert g.shape == u.shape and g.shape[0] == P
    inter = g.shape[1]
    w = np.ascontiguousarray(topk_w, np.float64).reshape(P)
    h = np.zeros((P, inter), np.float64)
    _load().orc_moe_v41_act(_ptr(g), _ptr(u), _ptr(w), _ptr(ids), P, inter,
                            float(swiglu_limit), _ptr(h))
    return h


def v41_routing(topk_ids, topk_w, n_experts, has_shared):
    """Routing with the shared expert as one more slot per token: expert
    n_experts with weight 1 (the banks then hold n_experts + 1 experts).
    Routed ids outside [0, n_experts) drop their pair and never select the
    shared expert."""
    ids = _sanitize_ids(topk_ids, n_experts)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    if not has_shared:
        return ids, w, n_experts
    T = ids.shape[0]
    ids2 = np.concatenate([ids, np.full((T, 1), n_experts, np.int32)], axis=1)
    w2 = np.concatenate([w, np.ones((T, 1), np.float32)], axis=1)
    return ids2, w2, n_experts + 1


def moe_v41(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w, swiglu_limit,
            has_shared, threads=None):
    """The V4.1 expert bank: per pair, exact gate/up products, the V4.1
    activation (bf16 gate/up, limit, route weight folded, bf16 h), the down
    product, then out[t] = sum over the token's slots of the down outputs
    (no further weighting), rounded once to bf16 ("cortiq-engine 0.8.40,
    src/gpu_wgpu/mxfp4.rs": dsv4_global_down_mxfp4 with its bf16 flag sums
    every slot of a token in one reduction).  With has_shared, expert
    n_experts is applied to every token with weight 1."""
    ids, w, E = v41_routing(topk_ids, topk_w, n_experts, has_shared)
    st = moe_gate_up(gate, up, E, hidden, inter, x, ids, False, threads)
    h = moe_v41_act(st["g"], st["u"], w, ids, E, swiglu_limit)
    y, mag_y = moe_down(down, E, hidden, inter, h, ids, threads)
    ones = np.ones(ids.shape, np.float64)
    out, mag_out = moe_combine(y, mag_y, ones, ids, E)
    st.update(h=h, y=y, mag_y=mag_y, out=out, mag_out=mag_out,
              out_bf16=bf16_rne_array(out).reshape(out.shape), ids=ids, w=w, n_experts=E)
    return st
