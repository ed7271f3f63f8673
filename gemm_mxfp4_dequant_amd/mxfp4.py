"""ctypes binding of ``libmxfp4.so`` (C ABI declared in ``include/mxfp4.h``).

Argument marshalling only: each function takes torch device tensors, passes
their data pointers, sizes and the current HIP stream to the C entry point of
the same name, and raises ``Mxfp4Error`` on a nonzero status.  Every step of
the computation runs in the library's HIP kernels; if the library is not
built, every call raises (there is no fallback).  Output tensors may be
given by the caller or are allocated here with torch.
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
        "moe_route_group": (I, [P, I64, I64, I64, P, P, P, P]),
        "moe_route_topk": (I, [P, I64, I64, I64, P, P, P]),
        "moe_experts_mxfp4_workspace_size": (ctypes.c_size_t, [I64, I64, I64, I64, I64, I]),
        "moe_experts_mxfp4": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I, P,
                                  ctypes.c_size_t, P]),
        "moe_experts_mxfp4_stages": (I, [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I,
                                         P, ctypes.c_size_t, P, P, P]),
        "moe_experts_mxfp4_v41_workspace_size": (ctypes.c_size_t, [I64, I64, I64, I64, I64, I]),
        "moe_experts_mxfp4_v41": (I, [P, P, P, I64, I64, I64, P, I64, P, P, I64,
                                      ctypes.c_float, I, P, P, ctypes.c_size_t, P]),
        "moe_experts_mxfp4_v41_stages": (I, [P, P, P, I64, I64, I64, P, I64, P, P, I64,
                                             ctypes.c_float, I, P, P, ctypes.c_size_t, P, P,
                                             P]),
        "mxfp4_last_error": (ctypes.c_char_p, []),
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


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


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
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=w.device)
    _check(lib().mxfp4_dequant(_ptr(w), rows, cols, _ptr(out), _dt(out), _stream(stream)))
    return out


def mxfp4_matvec(w, rows, cols, x, y=None, stream=None):
    if y is None:
        y = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().mxfp4_matvec(_ptr(w), rows, cols, _ptr(x), _ptr(y), _stream(stream)))
    return y


def mxfp4_gemm(w, rows, cols, x, b=None, y=None, y_dtype=torch.float32, stream=None):
    if b is None:
        b = x.shape[0]
    if y is None:
        y = torch.empty((b, rows), dtype=y_dtype, device=x.device)
    _check(lib().mxfp4_gemm(_ptr(w), rows, cols, _ptr(x), _dt(x), b, _ptr(y), _dt(y),
                            _stream(stream)))
    return y


def moe_route_group(topk_ids, n_experts, offsets=None, pair_of_slot=None, slot_of_pair=None,
                    stream=None):
    T, K = topk_ids.shape
    dev = topk_ids.device
    if offsets is None:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    if pair_of_slot is None:
        pair_of_slot = torch.full((T * K,), -1, dtype=torch.int32, device=dev)
    if slot_of_pair is None:
        slot_of_pair = torch.empty(T * K, dtype=torch.int32, device=dev)
    _check(lib().moe_route_group(_ptr(topk_ids), T, K, n_experts, _ptr(offsets),
                                 _ptr(pair_of_slot), _ptr(slot_of_pair), _stream(stream)))
    return offsets, pair_of_slot, slot_of_pair


def moe_route_topk(logits, top_k, topk_ids=None, topk_w=None, stream=None):
    """Top-k experts and renormalised weights of fp32 logits [T, E]."""
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check(lib().moe_route_topk(_ptr(logits), T, E, top_k, _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)))
    return topk_ids, topk_w


def moe_experts_mxfp4_workspace_size(n_tokens, top_k, n_experts, hidden, inter, x_dtype) -> int:
    code = x_dtype if isinstance(x_dtype, int) else (MXFP4_BF16 if x_dtype == torch.bfloat16
                                                     else MXFP4_F32)
    return int(lib().moe_experts_mxfp4_workspace_size(n_tokens, top_k, n_experts, hidden,
                                                      inter, code))


def _moe_ws(workspace, T, K, E, H, I, x, dev):
    need = moe_experts_mxfp4_workspace_size(T, K, E, H, I, _dt(x))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def moe_experts_mxfp4(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w, out=None,
                      out_dtype=torch.bfloat16, workspace=None, stream=None):
    T, K = topk_ids.shape
    if out is None:
        out = torch.empty((T, hidden), dtype=out_dtype, device=x.device)
    ws, ws_bytes = _moe_ws(workspace, T, K, n_experts, hidden, inter, x, x.device)
    _check(lib().moe_experts_mxfp4(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden, inter,
                                   _ptr(x), _dt(x), T, _ptr(topk_ids), _ptr(topk_w), K, _ptr(out),
                                   _dt(out), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def moe_experts_mxfp4_stages(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                             out=None, out_dtype=torch.bfloat16, workspace=None, h_in=None,
                             h_out=None, stream=None):
    T, K = topk_ids.shape
    ws, ws_bytes = _moe_ws(workspace, T, K, n_experts, hidden, inter, x, x.device)
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


def _v41_ws(workspace, T, K, E, H, I, has_shared, dev):
    need = moe_experts_mxfp4_v41_workspace_size(T, K, E, H, I, has_shared)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def moe_experts_mxfp4_v41(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                          swiglu_limit=0.0, has_shared=False, out=None, workspace=None,
                          stream=None):
    """V4.1 expert bank (bf16 x and out); with has_shared the banks hold
    n_experts + 1 experts, the shared one last."""
    T, K = topk_ids.shape
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    ws, ws_bytes = _v41_ws(workspace, T, K, n_experts, hidden, inter, has_shared, x.device)
    _check(lib().moe_experts_mxfp4_v41(_ptr(gate), _ptr(up), _ptr(down), n_experts, hidden,
                                       inter, _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), K,
                                       float(swiglu_limit), int(has_shared), _ptr(out), _ptr(ws),
                                       ws_bytes, _stream(stream)))
    return out


def moe_experts_mxfp4_v41_stages(gate, up, down, n_experts, hidden, inter, x, topk_ids, topk_w,
                                 swiglu_limit=0.0, has_shared=False, out=None, workspace=None,
                                 h_in=None, h_out=None, stream=None):
    T, K = topk_ids.shape
    ws, ws_bytes = _v41_ws(workspace, T, K, n_experts, hidden, inter, has_shared, x.device)
    _check(lib().moe_experts_mxfp4_v41_stages(_ptr(gate), _ptr(up), _ptr(down), n_experts,
                                              hidden, inter, _ptr(x), T, _ptr(topk_ids),
                                              _ptr(topk_w), K, float(swiglu_limit),
                                              int(has_shared), _ptr(out), _ptr(ws), ws_bytes,
                                              _ptr(h_in), _ptr(h_out), _stream(stream)))
    return out, h_out
