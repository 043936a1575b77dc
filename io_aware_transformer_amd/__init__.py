"""Python binding of the MI355X exact-attention library (libfa_fwd.so).

Argument marshalling only: every step of the forward and backward passes
runs in the HIP kernels behind the C ABI declared in include/fa_fwd.h and
include/fa_bwd.h.  PyTorch supplies device memory and streams.  There is no
fallback: if the library cannot be loaded (or built with hipcc), every call
raises.

C entry points mirrored here with the same names and argument order:
  fa_fwd_f16(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> status
  fa_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> status
  fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> status
  fa_fwd_window(q, k, v, o, lse, B, H, N, d, window_left, window_right, seqlens,
                scale, dtype, stream) -> status
  fa_fwd_split(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, ws,
               dtype, stream) -> status
  fa_fwd_split_noalloc(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits,
                       dtype, stream) -> status
  fa_fwd_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, ws,
                dtype, stream) -> status
  fa_fwd_decode_workspace_size(B, H, Nq, Nk, d, num_splits) -> bytes
  fa_fwd_decode_splits(B, H, Nq, Nk) -> segments
  fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, total, max_seqlen, d,
                causal, scale, dtype, stream) -> status
  fa_fwd_split_workspace_size(B, H, N, d, num_splits) -> bytes
  fa_bwd(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale,
         dtype, stream) -> status
  fa_bwd_workspace_size(B, H, N) -> bytes
  fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, p_drop, seed, offset,
                 dtype, stream) -> status
  fa_bwd_dropout(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale,
                 p_drop, seed, offset, dtype, stream) -> status
  fa_bwd_window(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, window_left,
                window_right, seqlens, scale, dtype, stream) -> status
  fa_bwd_varlen(q, k, v, o, dO, lse, cu_seqlens, ws, dq, dk, dv, B, H, total,
                max_seqlen, d, causal, scale, dtype, stream) -> status
  fa_bwd_varlen_workspace_size(B, H, total) -> bytes
  fa_status_string(status) -> str
Pointers may be given as integers or as tensors (their data_ptr()); the
stream as an integer handle, a torch.cuda.Stream, or None (null stream).
"""
from __future__ import annotations

import ctypes
from pathlib import Path

from .build import LIB as _LIB_PATH, build as _build

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_LAUNCH = -4
FA_ERR_SCRATCH = -5
FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1

EXPORTED = ("fa_fwd_f16", "fa_fwd_bf16", "fa_fwd", "fa_fwd_window", "fa_fwd_split",
            "fa_fwd_split_workspace_size", "fa_status_string", "fa_bwd",
            "fa_bwd_workspace_size", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_varlen",
            "fa_bwd_varlen", "fa_bwd_varlen_workspace_size", "fa_bwd_window",
            "fa_fwd_split_noalloc", "fa_fwd_decode", "fa_fwd_decode_workspace_size",
            "fa_fwd_decode_splits")
FA_MAX_SPLITS = 64
FA_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{fa_status_string(status)} (status {status})")


def library_path() -> Path:
    return _LIB_PATH


def load():
    """Load libfa_fwd.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        _build()
    lib = ctypes.CDLL(str(_LIB_PATH))
    p = ctypes.c_void_p
    i = ctypes.c_int
    f = ctypes.c_float
    sig = [p, p, p, p, p, i, i, i, i, i, f]
    lib.fa_fwd_f16.argtypes = sig + [p]
    lib.fa_fwd_bf16.argtypes = sig + [p]
    lib.fa_fwd.argtypes = sig + [i, p]
    for n in ("fa_fwd_f16", "fa_fwd_bf16", "fa_fwd"):
        getattr(lib, n).restype = ctypes.c_int
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd_window.argtypes = [p, p, p, p, p, i, i, i, i, i, i, p, f, i, p]
    lib.fa_fwd_window.restype = ctypes.c_int
    lib.fa_fwd_split.argtypes = [p, p, p, p, p, i, i, i, i, i, f, i, p, i, p]
    lib.fa_fwd_split.restype = ctypes.c_int
    lib.fa_fwd_split_noalloc.argtypes = [p, p, p, p, p, i, i, i, i, i, f, i, i, p]
    lib.fa_fwd_split_noalloc.restype = ctypes.c_int
    lib.fa_fwd_split_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_fwd_decode.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, i, p, i, p]
    lib.fa_fwd_decode.restype = ctypes.c_int
    lib.fa_fwd_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_decode_splits.argtypes = [i, i, i, i]
    lib.fa_fwd_decode_splits.restype = ctypes.c_int
    lib.fa_fwd_split_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [p] * 10 + [i, i, i, i, i, f, i, p]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_varlen.argtypes = [p, p, p, p, p, p, i, i, i, i, i, i, f, i, p]
    lib.fa_fwd_varlen.restype = ctypes.c_int
    u64 = ctypes.c_ulonglong
    u32 = ctypes.c_uint
    lib.fa_fwd_dropout.argtypes = sig + [f, u64, u32, i, p]
    lib.fa_fwd_dropout.restype = ctypes.c_int
    lib.fa_bwd_dropout.argtypes = [p] * 10 + [i, i, i, i, i, f, f, u64, u32, i, p]
    lib.fa_bwd_dropout.restype = ctypes.c_int
    lib.fa_bwd_window.argtypes = [p] * 10 + [i, i, i, i, i, i, p, f, i, p]
    lib.fa_bwd_window.restype = ctypes.c_int
    lib.fa_bwd_varlen.argtypes = [p] * 11 + [i, i, i, i, i, i, f, i, p]
    lib.fa_bwd_varlen.restype = ctypes.c_int
    lib.fa_bwd_varlen_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_varlen_workspace_size.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def fa_fwd_f16(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> int:
    return load().fa_fwd_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                             int(N), int(d), int(causal), float(scale), _stream(stream))


def fa_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> int:
    return load().fa_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                              int(N), int(d), int(causal), float(scale), _stream(stream))


def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream=None) -> int:
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                         int(N), int(d), int(causal), float(scale), int(dtype),
                         _stream(stream))


def fa_fwd_window(q, k, v, o, lse, B, H, N, d, window_left, window_right, seqlens, scale,
                  dtype, stream=None) -> int:
    return load().fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                int(N), int(d), int(window_left), int(window_right),
                                _ptr(seqlens), float(scale), int(dtype), _stream(stream))


def fa_fwd_split(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, ws, dtype,
                 stream=None) -> int:
    return load().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                               int(N), int(d), int(causal), float(scale), int(num_splits),
                               _ptr(ws), int(dtype), _stream(stream))


def fa_fwd_split_noalloc(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, dtype,
                         stream=None) -> int:
    return load().fa_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                       int(H), int(N), int(d), int(causal), float(scale),
                                       int(num_splits), int(dtype), _stream(stream))


def fa_fwd_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, ws, dtype,
                  stream=None) -> int:
    return load().fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                int(Nq), int(Nk), int(d), int(causal), float(scale),
                                int(num_splits), _ptr(ws), int(dtype), _stream(stream))


def fa_fwd_decode_workspace_size(B, H, Nq, Nk, d, num_splits) -> int:
    return int(load().fa_fwd_decode_workspace_size(int(B), int(H), int(Nq), int(Nk), int(d),
                                                   int(num_splits)))


def fa_fwd_decode_splits(B, H, Nq, Nk) -> int:
    return int(load().fa_fwd_decode_splits(int(B), int(H), int(Nq), int(Nk)))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, total, max_seqlen, d, causal, scale,
                  dtype, stream=None) -> int:
    return load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                _ptr(cu_seqlens), int(B), int(H), int(total), int(max_seqlen),
                                int(d), int(causal), float(scale), int(dtype), _stream(stream))


def fa_fwd_split_workspace_size(B, H, N, d, num_splits) -> int:
    return int(load().fa_fwd_split_workspace_size(int(B), int(H), int(N), int(d),
                                                  int(num_splits)))


def fa_bwd(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, dtype,
           stream=None) -> int:
    return load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(ws),
                         _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H), int(N), int(d),
                         int(causal), float(scale), int(dtype), _stream(stream))


def fa_bwd_workspace_size(B, H, N) -> int:
    return int(load().fa_bwd_workspace_size(int(B), int(H), int(N)))


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, p_drop, seed, offset, dtype,
                   stream=None) -> int:
    return load().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                 int(H), int(N), int(d), int(causal), float(scale),
                                 float(p_drop), int(seed), int(offset), int(dtype),
                                 _stream(stream))


def fa_bwd_dropout(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, p_drop,
                   seed, offset, dtype, stream=None) -> int:
    return load().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                 _ptr(ws), _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H),
                                 int(N), int(d), int(causal), float(scale), float(p_drop),
                                 int(seed), int(offset), int(dtype), _stream(stream))


def fa_bwd_window(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, window_left, window_right,
                  seqlens, scale, dtype, stream=None) -> int:
    return load().fa_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                _ptr(ws), _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H), int(N),
                                int(d), int(window_left), int(window_right), _ptr(seqlens),
                                float(scale), int(dtype), _stream(stream))


def fa_bwd_varlen(q, k, v, o, dO, lse, cu_seqlens, ws, dq, dk, dv, B, H, total, max_seqlen, d,
                  causal, scale, dtype, stream=None) -> int:
    return load().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                _ptr(cu_seqlens), _ptr(ws), _ptr(dq), _ptr(dk), _ptr(dv),
                                int(B), int(H), int(total), int(max_seqlen), int(d),
                                int(causal), float(scale), int(dtype), _stream(stream))


def fa_bwd_varlen_workspace_size(B, H, total) -> int:
    return int(load().fa_bwd_varlen_workspace_size(int(B), int(H), int(total)))


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def attention(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate o and lse for [B,H,N,d] CUDA tensors q, k, v and run the
    forward pass on `stream` (default: torch's current stream).
    Returns (o, lse); raises FaError on a non-zero status."""
    import torch
    if q.dtype == torch.float16:
        dt = FA_DTYPE_F16
    elif q.dtype == torch.bfloat16:
        dt = FA_DTYPE_BF16
    else:
        raise TypeError("q, k, v must be float16 or bfloat16")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,N,d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B,H,N,d]")
    if q.device.type != "cuda" or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU (there is no CPU path)")
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale, dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def attention_backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
                       stream=None):
    """Gradients (dq, dk, dv) of attention(q, k, v) for upstream gradient do,
    given the forward's o and lse.  Allocates the outputs and the workspace;
    raises FaError on a non-zero status."""
    import torch
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("q, k, v must be float16 or bfloat16")
    dt = FA_DTYPE_F16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B,H,N,d] tensor")
    for t in (k, v, o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("k, v, o, do must be contiguous and match q")
    # the kernel reads B*H*N fp32 row statistics from lse's first address
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32 (the forward's log-sum-exp)")
    if tuple(lse.shape) != tuple(q.shape[:3]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous [B,H,N] tensor")
    if any(t.device.type != "cuda" or t.device != q.device for t in (q, k, v, o, lse, do)):
        raise ValueError("all tensors must be on one GPU (there is no CPU path)")
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_bwd(q, k, v, o, do, lse, ws, dq, dk, dv, B, H, N, d, int(causal), scale, dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv
