"""ctypes binding of ``libmxfp4.so`` (C ABI declared in ``include/mxfp4.h``).

Argument marshalling only: each function takes torch device tensors, passes
their data pointers, sizes and the current HIP stream to the C entry point of
the same name, and raises ``Mxfp4Error`` on a nonzero status.  Every step of
the computation runs in the library's HIP kernels; if the library is not
built, every call raises (there is no fallback).  Output tensors may be
given by the caller or are allocated here with torch.

Before anything reaches the library, every tensor argument is checked here:
a device tensor on the current device, contiguous, of an accepted element
type, and at least as long as the sizes passed with it imply.  The C ABI
cannot see buffer lengths or memory kinds, so a host tensor or a short
buffer would otherwise reach a kernel.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4.so")

MXFP4_OK = 0
MXFP4_EINVAL = -1
MXFP4_EALIGN = -2
MXFP4_EWORKSPACE = -3
MXFP4_ELAUNCH = -4
MXFP4_F32 = 0
MXFP4_BF16 = 1

_lib = None


class Mxfp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "mxfp4_nbytes": (I64, [I64, I64]),
        "mxfp4_dequant": (I, [P, I64, I64, P, I, P]),
        "mxfp4_matvec": (I, [P, I64, I64, P, P, P]),
        "mxfp4_gemm": (I, [P, I64, I64, P, I, I64, P, I, P]),
        "mxfp8_quantize": (I, [P, I, I64, I64, P, P, P]),
        "mxfp4_gemm_a8_workspace_size": (ctypes.c_size_t, [I64, I64]),
        "mxfp4_gemm_a8": (I, [P, I64, I64, P, I, I64, P, I, P, ctypes.c_size_t, P]),
        "moe_route_group": (I, [P, I64, I64, I64, P, P, P, P]),
        "moe_route_topk": (I, [P, I64, I64, I64, P, P, P]),
        "moe_experts_mxfp4_workspace_size": (ctypes.c_size_t, [I64, I64, I64, I64, I64, I]),
        "moe_experts_mxfp4": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I, P,
                                  ctypes.c_size_t, P]),
        "moe_experts_mxfp4_stages": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I,
                                         P, ctypes.c_size_t, P, P, P]),
        "moe_experts_mxfp4_noalloc": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I,
                                          P]),
        "moe_experts_mxfp4_ptrs": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I, P,
                                       ctypes.c_size_t, P]),
        "moe_experts_mxfp4_a8_workspace_size": (ctypes.c_size_t, [I64, I64, I64, I64, I64]),
        "moe_experts_mxfp4_a8": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I, P,
                                     ctypes.c_size_t, P]),
        "mxfp4_device_address": (I, [P, ctypes.POINTER(ctypes.c_void_p)]),
        "moe_experts_mxfp4_v41_workspace_size": (ctypes.c_size_t, [I64, I64, I64, I64, I64, I]),
        "moe_experts_mxfp4_v41": (I, [P, P, P, I64, I64, I64, P, I64, P, P, I64,
                                      ctypes.c_float, I, P, P, ctypes.c_size_t, P]),
        "moe_experts_mxfp4_v41_stages": (I, [P, P, P, I64, I64, I64, P, I64, P, P, I64,
                                             ctypes.c_float, I, P, P, ctypes.c_size_t, P, P,
                                             P]),
        "mxfp4_last_error": (ctypes.c_char_p, []),
        "mxfp4_probe_read": (I, [P, I64, I, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != MXFP4_OK:
        raise Mxfp4Error(status, lib().mxfp4_last_error().decode())


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI sees raw pointers and sizes only, so this layer
# is the one place that can refuse a host tensor, a strided view, a wrong
# element type or a buffer shorter than the sizes claim, before a kernel
# would read or write outside it.
# ---------------------------------------------------------------------------

def _req(t, name, dtypes, numel=None, device=None):
    """Check one tensor argument; returns its device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device (cuda) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, other operands on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.dtype not in dtypes:
        names = ", ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{name}: dtype {str(t.dtype).replace('torch.', '')}, expected {names}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, needs at least {numel}")
    return t.device


def _req_shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _req_current(device):
    """Kernels are launched on the current device's stream: the operands must
    live there."""
    cur = torch.cuda.current_device()
    if device.index is not None and device.index != cur:
        raise ValueError(f"operands on {device}, current device is cuda:{cur}")


_ACT = (torch.float32, torch.bfloat16)
_U8 = (torch.uint8,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _sizes(**kw):
    for k, v in kw.items():
        if not isinstance(v, int) or isinstance(v, bool):
            raise TypeError(f"{k}: expected an int, got {type(v).__name__}")


def _tensor_bytes(rows, cols):
    n = mxfp4_nbytes(rows, cols)
    if n < 0:
        raise ValueError(f"rows = {rows}, cols = {cols}: not an MXFP4 shape (cols % 32 != 0)")
    return n


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MXFP4_F32
    if t.dtype == torch.bfloat16:
        return MXFP4_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dt(code: int):
    return torch.bfloat16 if code == MXFP4_BF16 else torch.float32


def mxfp4_nbytes(rows: int, cols: int) -> int:
    return int(lib().mxfp4_nbytes(rows, cols))


def mxfp4_last_error() -> str:
    return lib().mxfp4_last_error().decode()


def mxfp4_dequant(w, rows, cols, out=None, out_dtype=torch.float32, stream=None):
    _sizes(rows=rows, cols=cols)
    d = _req(w, "w", _U8, _tensor_bytes(rows, cols))
    _req_current(d)
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=w.device)
    _req(out, "out", _ACT, rows * cols, d)
    _check(lib().mxfp4_dequant(_ptr(w), rows, cols, _ptr(out), _dt(out), _stream(stream)))
    return out


def mxfp4_matvec(w, rows, cols, x, y=None, stream=None):
    _sizes(rows=rows, cols=cols)
    d = _req(w, "w", _U8, _tensor_bytes(rows, cols))
    _req_current(d)
    _req(x, "x", _F32, cols, d)
    if y is None:
        y = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _req(y, "y", _F32, rows, d)
    _check(lib().mxfp4_matvec(_ptr(w), rows, cols, _ptr(x), _ptr(y), _stream(stream)))
    return y


def mxfp4_gemm(w, rows, cols, x, b=None, y=None, y_dtype=torch.float32, stream=None):
    if b is None:
        b = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() >= 1 else 0
    _sizes(rows=rows, cols=cols, b=b)
    d = _req(w, "w", _U8, _tensor_bytes(rows, cols))
    _req_current(d)
    _req(x, "x", _ACT, b * cols, d)
    if y is None:
        y = torch.empty((b, rows), dtype=y_dtype, device=x.device)
    _req(y, "y", _ACT, b * rows, d)
    _check(lib().mxfp4_gemm(_ptr(w), rows, cols, _ptr(x), _dt(x), b, _ptr(y), _dt(y),
                            _stream(stream)))
    return y


def mxfp8_quantize(x, q=None, s=None, stream=None):
    """MXFP8 quantization of activations x [b, cols]: E4M3 codes q uint8
    [b, cols] and E8M0 scale bytes s uint8 [b, cols/32]."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x: expected a [b, cols] tensor")
    d = _req(x, "x", _ACT)
    _req_current(d)
    b, cols = x.shape
    if q is None:
        q = torch.empty((b, cols), dtype=torch.uint8, device=d)
    if s is None:
        s = torch.empty((b, cols // 32), dtype=torch.uint8, device=d)
    _req(q, "q", _U8, b * cols, d)
    _req(s, "s", _U8, b * (cols // 32), d)
    _check(lib().mxfp8_quantize(_ptr(x), _dt(x), b, cols, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def mxfp4_gemm_a8_workspace_size(b, cols) -> int:
    return int(lib().mxfp4_gemm_a8_workspace_size(b, cols))


def mxfp4_gemm_a8(w, rows, cols, x, b=None, y=None, y_dtype=torch.float32, workspace=None,
                  stream=None):
    """Opt-in block-scaled FP4 x FP8 GEMM (activations quantized to MXFP8;
    its own accuracy contract, see include/mxfp4.h)."""
    if b is None:
        b = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() >= 1 else 0
    _sizes(rows=rows, cols=cols, b=b)
    d = _req(w, "w", _U8, _tensor_bytes(rows, cols))
    _req_current(d)
    _req(x, "x", _ACT, b * cols, d)
    if y is None:
        y = torch.empty((b, rows), dtype=y_dtype, device=d)
    _req(y, "y", _ACT, b * rows, d)
    need = mxfp4_gemm_a8_workspace_size(b, cols)
    if need <= 0:
        raise ValueError(f"b = {b}, cols = {cols}: no FP4 x FP8 product (cols % 128 != 0?)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=d)
    _req(workspace, "workspace", _U8, need, d)
    _check(lib().mxfp4_gemm_a8(_ptr(w), rows, cols, _ptr(x), _dt(x), b, _ptr(y), _dt(y),
                               _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def _routing(topk_ids, d=None, topk_w=None):
    """Check the routing pair; returns (T, K, device)."""
    if not isinstance(topk_ids, torch.Tensor) or topk_ids.dim() != 2:
        raise ValueError("topk_ids: expected a [n_tokens, top_k] tensor")
    d = _req(topk_ids, "topk_ids", _I32, None, d)
    if topk_w is not None:
        _req(topk_w, "topk_w", _F32, None, d)
        _req_shape(topk_w, "topk_w", topk_ids.shape)
    T, K = topk_ids.shape
    return T, K, d


def moe_route_group(topk_ids, n_experts, offsets=None, pair_of_slot=None, slot_of_pair=None,
                    stream=None):
    _sizes(n_experts=n_experts)
    T, K, d = _routing(topk_ids)
    _req_current(d)
    if offsets is None:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=d)
    if pair_of_slot is None:
        pair_of_slot = torch.full((T * K,), -1, dtype=torch.int32, device=d)
    if slot_of_pair is None:
        slot_of_pair = torch.empty(T * K, dtype=torch.int32, device=d)
    _req(offsets, "offsets", _I32, n_experts + 1, d)
    _req(pair_of_slot, "pair_of_slot", _I32, T * K, d)
    _req(slot_of_pair, "slot_of_pair", _I32, T * K, d)
    _check(lib().moe_route_group(_ptr(topk_ids), T, K, n_experts, _ptr(offsets),
                                 _ptr(pair_of_slot), _ptr(slot_of_pair), _stream(stream)))
    return offsets, pair_of_slot, slot_of_pair


def moe_route_topk(logits, top_k, topk_ids=None, topk_w=None, stream=None):
    """Top-k experts and renormalised weights of fp32 logits [T, E]."""
    _sizes(top_k=top_k)
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits: expected a [n_tokens, n_experts] tensor")
    d = _req(logits, "logits", _F32)
    _req_current(d)
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=d)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=d)
    _req(topk_ids, "topk_ids", _I32, T * top_k, d)
    _req(topk_w, "topk_w", _F32, T * top_k, d)
    _check(lib().moe_route_topk(_ptr(logits), T, E, top_k, _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)))
    return topk_ids, topk_w


def moe_experts_mxfp4_workspace_size(n_tokens, top_k, n_experts, hidden, inter, x_dtype) -> int:
    code = x_dtype if isinstance(x_dtype, int) else (MXFP4_BF16 if x_dtype == torch.bfloat16
                                                     else MXFP4_F32)
    return int(lib().moe_experts_mxfp4_workspace_size(n_tokens, top_k, n_experts, hidden,
                                                      inter, code))


def _bank(gate, up, down, n_tensors, hidden, inter):
    """Check the three expert banks (n_tensors tensors per role); returns the
    device."""
    _sizes(hidden=hidden, inter=inter)
    tb = _tensor_bytes(inter, hidden)
    d = _req(gate, "gate", _U8, n_tensors * tb)
    _req(up, "up", _U8, n_tensors * tb, d)
    _req(down, "down", _U8, n_tensors * _tensor_bytes(hidden, inter), d)
    _req_current(d)
    return d


def _ws(workspace, need, d):
    if need <= 0:
        raise ValueError("expert bank sizes out of range (workspace size query returned 0)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=d)
    _req(workspace, "workspace", _U8, need, d)
    return workspace, workspace.numel()


def _h_buffers(h_in, h_out, n_slots, inter, dtypes, d):
    if h_in is not None:
        _req(h_in, "h_in", dtypes, n_slots * inter, d)
    if h_out is not None:
        _req(h_out, "h_out", dtypes, n_slots * inter, d)


def moe_experts_mxfp4(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w, out=None,
                      out_dtype=torch.bfloat16, workspace=None, stream=None):
    _sizes(n_experts=n_experts)
    d = _bank(gate, up, down, n_experts, hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _ACT, T * hidden, d)
    if out is None:
        out = torch.empty((T, hidden), dtype=out_dtype, device=d)
    _req(out, "out", _ACT, T * hidden, d)
    ws, ws_bytes = _ws(workspace, moe_experts_mxfp4_workspace_size(T, K, n_experts, hidden,
                                                                   inter, _dt(x)), d)
    _check(lib().moe_experts_mxfp4(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden, inter,
                                   _ptr(x), _dt(x), T, _ptr(topk_ids), _ptr(topk_w), K, _ptr(out),
                                   _dt(out), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def moe_experts_mxfp4_a8_workspace_size(n_tokens, top_k, n_experts, hidden, inter) -> int:
    return int(lib().moe_experts_mxfp4_a8_workspace_size(n_tokens, top_k, n_experts, hidden,
                                                         inter))


def moe_experts_mxfp4_a8(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                         out=None, out_dtype=torch.bfloat16, workspace=None, stream=None):
    """Opt-in expert bank on the block-scaled FP4 x FP8 product (x and h
    quantized to MXFP8; its own accuracy contract, see include/mxfp4.h)."""
    _sizes(n_experts=n_experts)
    d = _bank(gate, up, down, n_experts, hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _ACT, T * hidden, d)
    if out is None:
        out = torch.empty((T, hidden), dtype=out_dtype, device=d)
    _req(out, "out", _ACT, T * hidden, d)
    need = moe_experts_mxfp4_a8_workspace_size(T, K, n_experts, hidden, inter)
    if need <= 0:
        raise ValueError(f"hidden = {hidden}, inter = {inter}: no FP4 x FP8 expert bank "
                         "(multiples of 512 needed)")
    ws, ws_bytes = _ws(workspace, need, d)
    _check(lib().moe_experts_mxfp4_a8(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden,
                                      inter, _ptr(x), _dt(x), T, _ptr(topk_ids), _ptr(topk_w), K,
                                      _ptr(out), _dt(out), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def mxfp4_device_address(t) -> int:
    """Address kernels use for tensor ``t``'s data: a device tensor's own
    pointer, or the mapped address of a pinned host tensor.  Raises for
    pageable host memory."""
    out = ctypes.c_void_p()
    _check(lib().mxfp4_device_address(t.data_ptr(), ctypes.byref(out)))
    return int(out.value)


def expert_table(tensors, rows, cols, device=None):
    """Device table of per-expert tensor addresses for moe_experts_mxfp4_ptrs
    from a list of uint8 tensors, each either on the current device or in
    pinned host memory (``torch.empty(..., pin_memory=True)``)."""
    nb = _tensor_bytes(rows, cols)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    addrs = []
    for i, t in enumerate(tensors):
        name = f"expert {i}"
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor")
        if t.device.type == "cuda":
            _req(t, name, _U8, nb, dev)
        elif t.device.type == "cpu":
            if not t.is_pinned():
                raise ValueError(f"{name}: a host tensor must be in pinned memory")
            if not t.is_contiguous() or t.dtype != torch.uint8 or t.numel() < nb:
                raise ValueError(f"{name}: expected a contiguous uint8 tensor of {nb} bytes")
        else:
            raise ValueError(f"{name}: on {t.device}")
        a = mxfp4_device_address(t)
        if a % 16:
            raise ValueError(f"{name}: data not 16-byte aligned")
        addrs.append(a)
    return torch.tensor(addrs, dtype=torch.int64, device=dev)


def moe_experts_mxfp4_ptrs(gate_table, up_table, down_table, n_experts, hidden, inter, x,
                           topk_ids, topk_w, out=None, out_dtype=torch.bfloat16, workspace=None,
                           stream=None):
    """The expert bank over per-expert pointer tables (``expert_table``):
    each expert's tensors in device memory or pinned host memory."""
    _sizes(n_experts=n_experts, hidden=hidden, inter=inter)
    d = _req(gate_table, "gate_table", (torch.int64,), n_experts)
    _req(up_table, "up_table", (torch.int64,), n_experts, d)
    _req(down_table, "down_table", (torch.int64,), n_experts, d)
    _req_current(d)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _ACT, T * hidden, d)
    if out is None:
        out = torch.empty((T, hidden), dtype=out_dtype, device=d)
    _req(out, "out", _ACT, T * hidden, d)
    ws, ws_bytes = _ws(workspace, moe_experts_mxfp4_workspace_size(T, K, n_experts, hidden,
                                                                   inter, _dt(x)), d)
    _check(lib().moe_experts_mxfp4_ptrs(_ptr(gate_table), _ptr(up_table), _ptr(down_table),
                                        n_experts, hidden, inter, _ptr(x), _dt(x), T,
                                        _ptr(topk_ids), _ptr(topk_w), K, _ptr(out), _dt(out),
                                        _ptr(ws), ws_bytes, _stream(stream)))
    return out


MXFP4_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_experts_mxfp4_noalloc(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                              out, stream=None):
    """moe_experts_mxfp4 on the library's static device scratch (no
    workspace, nothing allocated by the library or here: ``out`` is the
    caller's).  Sizes needing more than MXFP4_NOALLOC_SCRATCH_BYTES of
    scratch are refused; calls that overlap on one GPU race."""
    _sizes(n_experts=n_experts)
    d = _bank(gate, up, down, n_experts, hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _ACT, T * hidden, d)
    _req(out, "out", _ACT, T * hidden, d)
    _check(lib().moe_experts_mxfp4_noalloc(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden,
                                           inter, _ptr(x), _dt(x), T, _ptr(topk_ids),
                                           _ptr(topk_w), K, _ptr(out), _dt(out),
                                           _stream(stream)))
    return out


def moe_experts_mxfp4_stages(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                             out=None, out_dtype=torch.bfloat16, workspace=None, h_in=None,
                             h_out=None, stream=None):
    _sizes(n_experts=n_experts)
    d = _bank(gate, up, down, n_experts, hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _ACT, T * hidden, d)
    if out is not None:
        _req(out, "out", _ACT, T * hidden, d)
    _h_buffers(h_in, h_out, T * K, inter, (x.dtype,), d)
    ws, ws_bytes = _ws(workspace, moe_experts_mxfp4_workspace_size(T, K, n_experts, hidden,
                                                                   inter, _dt(x)), d)
    out_code = _dt(out) if out is not None else (MXFP4_BF16 if out_dtype == torch.bfloat16
                                                 else MXFP4_F32)
    _check(lib().moe_experts_mxfp4_stages(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden,
                                          inter, _ptr(x), _dt(x), T, _ptr(topk_ids),
                                          _ptr(topk_w), K, _ptr(out), out_code, _ptr(ws),
                                          ws_bytes, _ptr(h_in), _ptr(h_out), _stream(stream)))
    return out, h_out


def moe_experts_mxfp4_v41_workspace_size(n_tokens, top_k, n_experts, hidden, inter,
                                         has_shared) -> int:
    return int(lib().moe_experts_mxfp4_v41_workspace_size(n_tokens, top_k, n_experts, hidden,
                                                          inter, int(has_shared)))


_BF16 = (torch.bfloat16,)


def moe_experts_mxfp4_v41(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                          swiglu_limit=0.0, has_shared=False, out=None, workspace=None,
                          stream=None):
    """V4.1 expert bank (bf16 x and out); with has_shared the banks hold
    n_experts + 1 experts, the shared one last."""
    _sizes(n_experts=n_experts)
    d = _bank(gate, up, down, n_experts + int(bool(has_shared)), hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _BF16, T * hidden, d)
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=d)
    _req(out, "out", _BF16, T * hidden, d)
    ws, ws_bytes = _ws(workspace, moe_experts_mxfp4_v41_workspace_size(
        T, K, n_experts, hidden, inter, has_shared), d)
    _check(lib().moe_experts_mxfp4_v41(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden,
                                       inter, _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), K,
                                       float(swiglu_limit), int(has_shared), _ptr(out), _ptr(ws),
                                       ws_bytes, _stream(stream)))
    return out


def moe_experts_mxfp4_v41_stages(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                                 swiglu_limit=0.0, has_shared=False, out=None, workspace=None,
                                 h_in=None, h_out=None, stream=None):
    _sizes(n_experts=n_experts)
    sh = int(bool(has_shared))
    d = _bank(gate, up, down, n_experts + sh, hidden, inter)
    T, K, _ = _routing(topk_ids, d, topk_w)
    _req(x, "x", _BF16, T * hidden, d)
    if out is not None:
        _req(out, "out", _BF16, T * hidden, d)
    _h_buffers(h_in, h_out, T * (K + sh), inter, _BF16, d)
    ws, ws_bytes = _ws(workspace, moe_experts_mxfp4_v41_workspace_size(
        T, K, n_experts, hidden, inter, has_shared), d)
    _check(lib().moe_experts_mxfp4_v41_stages(_ptr(gate), _ptr(up), _ptr(down), n_experts,
                                              hidden, inter, _ptr(x), T, _ptr(topk_ids),
                                              _ptr(topk_w), K, float(swiglu_limit),
                                              int(has_shared), _ptr(out), _ptr(ws), ws_bytes,
                                              _ptr(h_in), _ptr(h_out), _stream(stream)))
    return out, h_out


def mxfp4_probe_read(buf, nbytes=None, loads_per_thread=8, sink=None, stream=None):
    """Measurement helper: one streaming read of ``nbytes`` bytes of ``buf``
    (default: all of it).  Writes nothing."""
    d = _req(buf, "buf", _U8)
    _req_current(d)
    nbytes = buf.numel() if nbytes is None else nbytes
    _sizes(nbytes=nbytes, loads_per_thread=loads_per_thread)
    if nbytes > buf.numel():
        raise ValueError(f"buf: {buf.numel()} bytes, {nbytes} requested")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=d)
    _req(sink, "sink", (torch.int32,), 1, d)
    st = lib().mxfp4_probe_read(_ptr(buf), nbytes, loads_per_thread, _ptr(sink), _stream(stream))
    if st != 0:
        raise Mxfp4Error(st, "mxfp4_probe_read refused its arguments")
