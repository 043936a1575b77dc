"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the oracle shares
no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module builds it with gcc and marshals numpy arrays through ctypes.  Inputs
are raw 16-bit bit patterns (``numpy.uint16``) in [B,H,N,d] order, so the
oracle sees exactly the bits the GPU sees.

Pages cited (by tag and section):
  [P-notes] "FlashAttention v1 & v2 笔记" (yiran529.github.io)
  [P-baidu] "FlashAttention 优化原理与实现要点解析" (cloud.baidu.com)
  [P-wmrh]  "FlashAttention V2 核心原理与架构设计" (wmrh.cn)

Functions and what pins them (tests/test_oracle.py):
  attn_fwd        plain definition, [P-baidu] §1, §2, §4.1 -- brute force vs a
                  library softmax, invariants, closed forms
  attn_fwd_rows   the same on selected rows -- agreement with attn_fwd
  attn_fwd_varlen packed variable-length sequences (the padding / varlen
                  mask kinds of [P-baidu] §8): attn_fwd on every sequence --
                  a batch of equal lengths against attn_fwd on [B,H,N,d]
  attn_bwd_varlen its gradients: attn_bwd (given o) on every sequence -- the
                  same batched comparison
  attn_probs      P = Softmax(S) -- rows sum to 1, brute force
  attn_fwd_tiled  block algorithm of [P-baidu] §4.2-§6 -- agreement with
                  attn_fwd at several tile sizes
  softmax_1d / softmax_online_1d  [P-baidu] §4.1 / [P-wmrh] §2.1 -- library
                  softmax and each other
  attn_bwd        gradients dQ, dK, dV of the plain definition for an upstream
                  dO (chain rule; the pages print no gradient formulas) --
                  torch fp64 autograd, central differences of a pure-Python
                  forward, closed-form invariants (sum_j dK_j = 0,
                  sum_j dV_j = sum_i dO_i, constant V, causal row 0)
                  With a given 16-bit o the row term is dO . o (as a backward
                  pass fed the forward's output computes it) -- pinned by the
                  exact linear shift it causes (dq by -scale dD (P K), dk by
                  -scale P^T (dD q), dv unchanged)
  attn_bwd_rows   the same on sampled query rows (dQ) and key rows (dK, dV)
                  -- agreement with attn_bwd
  philox4x32_10   the counter-based generator (SC 2011 definition) -- the
                  published known-answer vectors (tests/golden)
  dropout_factors keep factors Z_ij (256/T or 0) of the documented mapping
                  -- the mapping re-derived from philox4x32_10, keep rate
  attn_fwd_dropout / attn_bwd_dropout  attention with dropout after the
                  softmax -- p = 0 reproduces attn_fwd / attn_bwd(o), torch
                  fp64 with an explicit keep matrix, autograd up to the exact
                  shift of the given-o row term
  attn_fwd_masked sliding window (wl, wr) and per-batch valid lengths
                  ([P-baidu] §8 mask kinds) -- the unmasked and causal cases
                  of attn_fwd, padded batches against their unpadded slices,
                  library softmax with an explicit mask matrix
  attn_fwd_decode Nq query rows against Nk keys, causal aligned bottom-right
                  (FlashDecoding shapes, [P-wmrh] §5.1) -- a library softmax
                  with an explicit mask, the square case of attn_fwd, the last
                  rows of a square causal problem, Q = 0 and constant-V
                  closed forms
  decode          binary16 / bfloat16 decoders -- all 65536 patterns vs a
                  library cast, hand-checked values
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "oracle.c"
_LIB = _DIR / "liboracle.so"

DTYPE_F16 = 0
DTYPE_BF16 = 1

_default = None


def build(force: bool = True, src: Path = _SRC, out: Path = _LIB) -> Path:
    """Compile oracle.c into a shared library with gcc (fp64, no fast-math)."""
    if not force and out.exists():
        return out
    tmp = out.with_suffix(".so.tmp")
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-std=c11", "-Wall", "-shared", "-fPIC", str(src), "-o", str(tmp), "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    f64 = ctypes.c_double
    lib.oracle_decode.argtypes = [p, i32, i64, p]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_softmax_1d.argtypes = [p, i64, p]
    lib.oracle_softmax_online_1d.argtypes = [p, i64, p]
    lib.oracle_attn_fwd.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64, p, p]
    lib.oracle_attn_fwd_rows.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64,
                                         p, i64, p, p]
    lib.oracle_attn_probs.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64, p]
    lib.oracle_attn_fwd_tiled.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64,
                                          i64, i64, p, p]
    lib.oracle_attn_bwd.argtypes = [p, p, p, p, p, i32, i64, i64, i64, i64, i32, f64, p, p, p]
    lib.oracle_attn_bwd_rows.argtypes = [p, p, p, p, p, i32, i64, i64, i64, i64, i32, f64,
                                         p, i64, p, i64, p, p, p]
    lib.oracle_attn_fwd_masked.argtypes = [p, p, p, i32, i64, i64, i64, i64, i64, i64, p,
                                           f64, p, p]
    lib.oracle_attn_fwd_decode.argtypes = [p, p, p, i32, i64, i64, i64, i64, i64, i32, f64,
                                           p, p]
    lib.oracle_attn_bwd_masked.argtypes = [p, p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                           p, f64, p, p, p]
    u64 = ctypes.c_uint64
    u32 = ctypes.c_uint32
    lib.oracle_philox4x32_10.argtypes = [p, p, p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_dropout_factors.argtypes = [i64, i64, u64, u32, i32, p]
    lib.oracle_attn_fwd_dropout.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64, i32,
                                            u64, u32, p, p]
    lib.oracle_attn_bwd_dropout.argtypes = [p, p, p, p, p, i32, i64, i64, i64, i64, i32, f64,
                                            i32, u64, u32, p, p, p]
    lib.oracle_attn_fwd_dropout_rows.argtypes = [p, p, p, i32, i64, i64, i64, i64, i32, f64,
                                                 i32, u64, u32, p, i64, p, p]
    lib.oracle_attn_bwd_dropout_rows.argtypes = [p, p, p, p, p, i32, i64, i64, i64, i64, i32,
                                                 f64, i32, u64, u32, p, i64, p, i64, p, p, p]
    for name in ("oracle_decode", "oracle_num_threads", "oracle_attn_fwd",
                 "oracle_attn_fwd_rows", "oracle_attn_probs", "oracle_attn_fwd_tiled",
                 "oracle_attn_bwd", "oracle_attn_bwd_rows", "oracle_attn_fwd_masked",
                 "oracle_attn_bwd_masked", "oracle_attn_fwd_decode",
                 "oracle_dropout_factors", "oracle_attn_fwd_dropout", "oracle_attn_bwd_dropout",
                 "oracle_attn_fwd_dropout_rows", "oracle_attn_bwd_dropout_rows"):
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_softmax_1d.restype = None
    lib.oracle_softmax_online_1d.restype = None
    return lib


def _load():
    global _default
    if _default is None:
        if not _LIB.exists():
            build()
        _default = Oracle(_LIB)
    return _default._lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are raw 16-bit patterns (numpy.uint16)")
    return x


def _dtype_code(dtype) -> int:
    if dtype in (DTYPE_F16, "f16", "fp16", "float16"):
        return DTYPE_F16
    if dtype in (DTYPE_BF16, "bf16", "bfloat16"):
        return DTYPE_BF16
    raise ValueError(f"unknown dtype {dtype!r}")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def _impl_num_threads(lib) -> int:
    return int(lib.oracle_num_threads())


def _impl_decode(lib, bits: np.ndarray, dtype) -> np.ndarray:
    bits = _bits(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(lib.oracle_decode(_ptr(bits), _dtype_code(dtype), bits.size, _ptr(out)),
           "oracle_decode")
    return out


def _impl_softmax_1d(lib, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib.oracle_softmax_1d(_ptr(x), x.size, _ptr(out))
    return out


def _impl_softmax_online_1d(lib, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib.oracle_softmax_online_1d(_ptr(x), x.size, _ptr(out))
    return out


def _shape(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B,H,N,d] shape")
    return q.shape


def _impl_attn_fwd(lib, q, k, v, dtype, causal: bool, scale: float):
    """Exact attention in fp64.  Returns (o [B,H,N,d], lse [B,H,N])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype),
                               B, H, N, d, int(bool(causal)), float(scale),
                               _ptr(o), _ptr(lse)), "oracle_attn_fwd")
    return o, lse


def _impl_attn_fwd_rows(lib, q, k, v, dtype, causal: bool, scale: float, rows):
    """Exact attention on selected flat rows (b*H+h)*N+i.
    Returns (o [n_rows,d], lse [n_rows])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    _check(lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype),
                                    B, H, N, d, int(bool(causal)), float(scale),
                                    _ptr(rows), rows.size, _ptr(o), _ptr(lse)),
           "oracle_attn_fwd_rows")
    return o, lse


def _impl_attn_probs(lib, q, k, v, dtype, causal: bool, scale: float):
    """The attention weights P [B,H,N,N] (masked entries 0).  Tiny inputs."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    p = np.empty((B, H, N, N), dtype=np.float64)
    _check(lib.oracle_attn_probs(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype),
                                 B, H, N, d, int(bool(causal)), float(scale), _ptr(p)),
           "oracle_attn_probs")
    return p


def _impl_attn_fwd_tiled(lib, q, k, v, dtype, causal: bool, scale: float,
                         Br: int, Bc: int):
    """The block algorithm (online-softmax merge) in fp64."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(lib.oracle_attn_fwd_tiled(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype),
                                     B, H, N, d, int(bool(causal)), float(scale),
                                     int(Br), int(Bc), _ptr(o), _ptr(lse)),
           "oracle_attn_fwd_tiled")
    return o, lse


def _given_o(o, shape):
    if o is None:
        return None
    o = _bits(o)
    if o.shape != shape:
        raise ValueError("o must have the [B,H,N,d] shape of q")
    return o


def _impl_attn_bwd(lib, q, k, v, do, dtype, causal: bool, scale: float, o=None):
    """Gradients of the exact attention for upstream gradient do, in fp64.
    With o (16-bit bits of a forward output) the row term is dO_i . o_i.
    Returns (dq, dk, dv), each [B,H,N,d]."""
    q, k, v, do = _bits(q), _bits(k), _bits(v), _bits(do)
    B, H, N, d = _shape(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have the [B,H,N,d] shape of q")
    o = _given_o(o, q.shape)
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    _check(lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do),
                               None if o is None else _ptr(o), _dtype_code(dtype),
                               B, H, N, d, int(bool(causal)), float(scale),
                               _ptr(dq), _ptr(dk), _ptr(dv)), "oracle_attn_bwd")
    return dq, dk, dv


def _impl_attn_bwd_rows(lib, q, k, v, do, dtype, causal: bool, scale: float,
                        qrows, krows, o=None):
    """dq on flat query rows qrows and (dk, dv) on flat key rows krows
    ((b*H+h)*N+i), optionally with the row term from a given o.
    Returns (dq [n_q,d], dk [n_k,d], dv [n_k,d])."""
    q, k, v, do = _bits(q), _bits(k), _bits(v), _bits(do)
    B, H, N, d = _shape(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have the [B,H,N,d] shape of q")
    o = _given_o(o, q.shape)
    qrows = np.ascontiguousarray(qrows, dtype=np.int64)
    krows = np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.empty((qrows.size, d), dtype=np.float64)
    dk = np.empty((krows.size, d), dtype=np.float64)
    dv = np.empty((krows.size, d), dtype=np.float64)
    _check(lib.oracle_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                    None if o is None else _ptr(o), _dtype_code(dtype),
                                    B, H, N, d, int(bool(causal)), float(scale),
                                    _ptr(qrows), qrows.size, _ptr(krows), krows.size,
                                    _ptr(dq), _ptr(dk), _ptr(dv)), "oracle_attn_bwd_rows")
    return dq, dk, dv


def _impl_attn_fwd_masked(lib, q, k, v, dtype, window_left: int, window_right: int,
                          seqlens, scale: float):
    """Attention with a sliding window and optional per-batch valid lengths
    (seqlens: B ints or None).  Rows without keys: o = 0, lse = -inf.
    Returns (o [B,H,N,d], lse [B,H,N])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    sl = None
    if seqlens is not None:
        sl = np.ascontiguousarray(seqlens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seqlens must hold one length per batch element")
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(lib.oracle_attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype), B, H, N,
                                      d, int(window_left), int(window_right),
                                      None if sl is None else _ptr(sl), float(scale),
                                      _ptr(o), _ptr(lse)), "oracle_attn_fwd_masked")
    return o, lse


def _impl_attn_fwd_decode(lib, q, k, v, dtype, causal: bool, scale: float):
    """Nq query rows (q: [B,H,Nq,d]) against Nk keys (k, v: [B,H,Nk,d]);
    causal: query i uses keys j <= i + Nk - Nq.  Rows without keys: o = 0,
    lse = -inf.  Returns (o [B,H,Nq,d], lse [B,H,Nq])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B,H,Nq,d]; k and v one [B,H,Nk,d] shape")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("q, k, v must share B, H and d")
    Nk = k.shape[2]
    o = np.empty((B, H, Nq, d), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    _check(lib.oracle_attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype), B, H, Nq,
                                      Nk, d, int(bool(causal)), float(scale), _ptr(o),
                                      _ptr(lse)), "oracle_attn_fwd_decode")
    return o, lse


def _impl_attn_bwd_masked(lib, q, k, v, do, dtype, window_left: int, window_right: int,
                          seqlens, scale: float, o=None):
    """Gradients of attn_fwd_masked (same window and lengths) for upstream
    do, in fp64; with o (16-bit bits of a forward output) the row term is
    dO_i . o_i.  Rows without keys add nothing.  Returns (dq, dk, dv), each
    [B,H,N,d]."""
    q, k, v, do = _bits(q), _bits(k), _bits(v), _bits(do)
    B, H, N, d = _shape(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have the [B,H,N,d] shape of q")
    o = _given_o(o, q.shape)
    sl = None
    if seqlens is not None:
        sl = np.ascontiguousarray(seqlens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seqlens must hold one length per batch element")
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    _check(lib.oracle_attn_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                      None if o is None else _ptr(o), _dtype_code(dtype),
                                      B, H, N, d, int(window_left), int(window_right),
                                      None if sl is None else _ptr(sl), float(scale),
                                      _ptr(dq), _ptr(dk), _ptr(dv)), "oracle_attn_bwd_masked")
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, dtype, cu_seqlens, causal: bool, scale: float):
    """Attention over packed variable-length sequences: q, k, v are uint16
    bit patterns [H, total, d]; sequence b holds tokens cu_seqlens[b] ..
    cu_seqlens[b+1]-1 of every head, and attends only within itself (causal
    or not, top-left aligned).  By definition each sequence is an
    independent attention problem, so this runs attn_fwd on every
    (head, sequence) slice.  Returns o [H, total, d] and lse [H, total]
    (fp64); tokens outside every sequence (after cu_seqlens[-1]) are 0 and
    -inf."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v))
    if q.ndim != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [H, total, d] shape")
    H, total, d = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > total:
        raise ValueError("cu_seqlens must rise from 0 to at most total")
    o = np.zeros((H, total, d), dtype=np.float64)
    lse = np.full((H, total), -np.inf, dtype=np.float64)
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        sl = lambda x: np.ascontiguousarray(x[:, lo:hi, :][None])
        ob, lb = attn_fwd(sl(q), sl(k), sl(v), dtype, causal, scale)
        o[:, lo:hi, :] = ob[0]
        lse[:, lo:hi] = lb[0]
    return o, lse


def attn_bwd_varlen(q, k, v, do, o, dtype, cu_seqlens, causal: bool, scale: float):
    """Gradients of attn_fwd_varlen for an upstream do, with the row term
    from the given 16-bit o (as attn_bwd(..., o=...)): every sequence is an
    independent problem, so this runs attn_bwd on every (head, sequence)
    slice.  All arrays [H, total, d]; rows outside every sequence get 0."""
    arrs = [np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v, do, o)]
    q, k, v, do, o = arrs
    if q.ndim != 3 or any(x.shape != q.shape for x in arrs):
        raise ValueError("q, k, v, do, o must share one [H, total, d] shape")
    H, total, d = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > total:
        raise ValueError("cu_seqlens must rise from 0 to at most total")
    grads = [np.zeros((H, total, d), dtype=np.float64) for _ in range(3)]
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        sl = lambda x: np.ascontiguousarray(x[:, lo:hi, :][None])
        gb = attn_bwd(sl(q), sl(k), sl(v), sl(do), dtype, causal, scale, o=sl(o))
        for g, x in zip(grads, gb):
            g[:, lo:hi, :] = x[0]
    return tuple(grads)


def dropout_threshold(p_drop: float) -> int:
    """T = round((1 - p) * 256): a weight is kept when its byte is below T."""
    if not (0.0 <= p_drop < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(np.floor((1.0 - p_drop) * 256.0 + 0.5))


def _impl_philox4x32_10(lib, counter, key):
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    kk = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(kk), _ptr(out))
    return out


def _impl_dropout_factors(lib, BH: int, N: int, seed: int, offset: int, T: int):
    """Z [BH, N, N]: 256/T where element (bh, i, j) is kept, else 0."""
    z = np.empty((BH, N, N), dtype=np.float64)
    _check(lib.oracle_dropout_factors(BH, N, int(seed), int(offset), int(T), _ptr(z)),
           "oracle_dropout_factors")
    return z


def _impl_attn_fwd_dropout(lib, q, k, v, dtype, causal: bool, scale: float, T: int, seed: int,
                           offset: int):
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(lib.oracle_attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype), B, H, N,
                                       d, int(bool(causal)), float(scale), int(T), int(seed),
                                       int(offset), _ptr(o), _ptr(lse)),
           "oracle_attn_fwd_dropout")
    return o, lse


def _impl_attn_bwd_dropout(lib, q, k, v, do, o, dtype, causal: bool, scale: float, T: int,
                           seed: int, offset: int):
    q, k, v, do = _bits(q), _bits(k), _bits(v), _bits(do)
    B, H, N, d = _shape(q, k, v)
    o = _given_o(o, q.shape)
    if o is None:
        raise ValueError("the dropout backward takes the row term from a given o")
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    _check(lib.oracle_attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(o),
                                       _dtype_code(dtype), B, H, N, d, int(bool(causal)),
                                       float(scale), int(T), int(seed), int(offset),
                                       _ptr(dq), _ptr(dk), _ptr(dv)), "oracle_attn_bwd_dropout")
    return dq, dk, dv


def _impl_attn_fwd_dropout_rows(lib, q, k, v, dtype, causal: bool, scale: float, T: int,
                                seed: int, offset: int, rows):
    """attn_fwd_dropout on selected flat rows (b*H+h)*N+i.
    Returns (o [n_rows,d], lse [n_rows])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, H, N, d = _shape(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    _check(lib.oracle_attn_fwd_dropout_rows(_ptr(q), _ptr(k), _ptr(v), _dtype_code(dtype), B, H,
                                            N, d, int(bool(causal)), float(scale), int(T),
                                            int(seed), int(offset), _ptr(rows), rows.size,
                                            _ptr(o), _ptr(lse)),
           "oracle_attn_fwd_dropout_rows")
    return o, lse


def _impl_attn_bwd_dropout_rows(lib, q, k, v, do, o, dtype, causal: bool, scale: float, T: int,
                                seed: int, offset: int, qrows, krows):
    """attn_bwd_dropout (o given) on flat query rows qrows (dq) and flat key
    rows krows (dk, dv).  Returns (dq [n_q,d], dk [n_k,d], dv [n_k,d])."""
    q, k, v, do = _bits(q), _bits(k), _bits(v), _bits(do)
    B, H, N, d = _shape(q, k, v)
    o = _given_o(o, q.shape)
    if o is None:
        raise ValueError("the dropout backward takes the row term from a given o")
    qrows = np.ascontiguousarray(qrows, dtype=np.int64)
    krows = np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.empty((qrows.size, d), dtype=np.float64)
    dk = np.empty((krows.size, d), dtype=np.float64)
    dv = np.empty((krows.size, d), dtype=np.float64)
    _check(lib.oracle_attn_bwd_dropout_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(o),
                                            _dtype_code(dtype), B, H, N, d, int(bool(causal)),
                                            float(scale), int(T), int(seed), int(offset),
                                            _ptr(qrows), qrows.size, _ptr(krows), krows.size,
                                            _ptr(dq), _ptr(dk), _ptr(dv)),
           "oracle_attn_bwd_dropout_rows")
    return dq, dk, dv


_API = ("num_threads", "decode", "softmax_1d", "softmax_online_1d", "attn_fwd",
        "attn_fwd_rows", "attn_probs", "attn_fwd_tiled", "attn_bwd", "attn_bwd_rows",
        "attn_fwd_masked", "attn_bwd_masked", "attn_fwd_decode", "philox4x32_10", "dropout_factors",
        "attn_fwd_dropout", "attn_bwd_dropout", "attn_fwd_dropout_rows",
        "attn_bwd_dropout_rows")


class Oracle:
    """One loaded build of oracle.c, with the functions of this module as
    methods.  The module-level functions use the default build; tests that
    plant mistakes load a mutated copy through this class."""

    def __init__(self, path):
        self._lib = _bind(ctypes.CDLL(str(path)))

    def __getattr__(self, name):
        if name not in _API:
            raise AttributeError(name)
        fn = globals()["_impl_" + name]
        return lambda *a, **kw: fn(self._lib, *a, **kw)


def _module_fn(name):
    impl = globals()["_impl_" + name]

    def fn(*a, **kw):
        return impl(_load(), *a, **kw)

    fn.__name__ = name
    fn.__doc__ = impl.__doc__
    return fn


num_threads = _module_fn("num_threads")
decode = _module_fn("decode")
softmax_1d = _module_fn("softmax_1d")
softmax_online_1d = _module_fn("softmax_online_1d")
attn_fwd = _module_fn("attn_fwd")
attn_fwd_rows = _module_fn("attn_fwd_rows")
attn_probs = _module_fn("attn_probs")
attn_fwd_tiled = _module_fn("attn_fwd_tiled")
attn_bwd = _module_fn("attn_bwd")
attn_bwd_rows = _module_fn("attn_bwd_rows")
attn_fwd_masked = _module_fn("attn_fwd_masked")
attn_bwd_masked = _module_fn("attn_bwd_masked")
attn_fwd_decode = _module_fn("attn_fwd_decode")
philox4x32_10 = _module_fn("philox4x32_10")
dropout_factors = _module_fn("dropout_factors")
attn_fwd_dropout = _module_fn("attn_fwd_dropout")
attn_bwd_dropout = _module_fn("attn_bwd_dropout")
attn_fwd_dropout_rows = _module_fn("attn_fwd_dropout_rows")
attn_bwd_dropout_rows = _module_fn("attn_bwd_dropout_rows")
