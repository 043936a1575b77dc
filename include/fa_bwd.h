/*
 * fa_bwd.h -- C ABI of the MI355X (gfx950) exact-attention backward pass.
 *
 * Operation.  For the forward o = Softmax(scale * q k^T) v of fa_fwd.h and
 * an upstream gradient dO of o, per batch b and head h:
 *     P_ij  = exp(scale * q_i . k_j - lse_i)        (j allowed for i, else 0)
 *     dV_j  = sum_i P_ij dO_i
 *     dS_ij = P_ij (dO_i . v_j - D_i),   D_i = dO_i . o_i
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_i dS_ij q_i
 * with the allowed keys of fa_fwd (all, or j <= i when causal).  This is the
 * chain rule through Attention(Q,K,V) = Softmax(Q K^T / sqrt(d)) V of
 * "FlashAttention 优化原理与实现要点解析" (cloud.baidu.com) §1; the per-row
 * statistics that page keeps apart for the backward pass (§6, numerator and
 * denominator) arrive here as lse, the fp32 logsumexp fa_fwd writes, so P is
 * recomputed tile by tile and never stored.  D_i = dO_i . o_i equals
 * sum_j P_ij (dO_i . v_j) because o_i = sum_j P_ij v_j.
 *
 * Layout.  q, k, v, o, dO, dq, dk, dv are contiguous [B,H,N,d] arrays of one
 * 16-bit type (binary16 or bfloat16), element (b,h,n,c) at
 * ((b*H+h)*N+n)*d+c; lse is fp32 [B,H,N].  Accumulation is fp32; P and dS
 * are rounded to the input type (nearest-even) as MFMA operands; dq, dk, dv
 * are rounded to the input type once, at the end.
 *
 * Ownership.  All pointers are device pointers owned by the caller.  ws is a
 * caller-owned fp32 workspace of fa_bwd_workspace_size(B, H, N) bytes; the
 * call overwrites it (its contents afterwards are unspecified).  The library
 * allocates nothing and keeps no state between calls.  q, k, v, o, dO and lse
 * are only read; dq, dk and dv are fully overwritten.  No output or ws may
 * overlap an input or another output.
 *
 * Errors.  As fa_fwd: arguments are validated on the host before any HIP
 * call, and a failing call touches no memory.  A passing call enqueues three
 * kernels on `stream` and returns without waiting.  Results are
 * deterministic (no atomics): the same inputs give the same bits.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stddef.h>
#include "fa_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of fp32 workspace fa_bwd needs for B*H heads of N rows (0 if the
 * sizes are not positive). */
size_t fa_bwd_workspace_size(int B, int H, int N);

/* Backward pass:
 *   q, k, v, o, dO  [B,H,N,d] 16-bit (o and lse as written by fa_fwd for the
 *                   same q, k, v, causal and scale), read only
 *   lse             [B,H,N] fp32 (natural log), read only
 *   ws              fa_bwd_workspace_size(B,H,N) bytes, 16-byte aligned,
 *                   scratch
 *   dq, dk, dv      [B,H,N,d] 16-bit, written
 *   B, H, N, d, causal, scale, dtype: as fa_fwd (d 64 or 128)
 * Returns FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED / FA_ERR_MISALIGNED /
 * FA_ERR_LAUNCH under the same rules as fa_fwd (ws must be 16-byte aligned). */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o,
                 const void *dO, const float *lse, float *ws, void *dq, void *dk,
                 void *dv, int B, int H, int N, int d, int causal, float scale,
                 fa_dtype dtype, hipStream_t stream);

/* Backward pass of fa_fwd_dropout: the same gradients for
 *     o_i = sum_j P_ij Z_ij v_j      (Z the keep factors of fa_fwd_dropout)
 * namely
 *     dV_j  = sum_i P_ij Z_ij dO_i
 *     dS_ij = P_ij (Z_ij (dO_i . v_j) - D_i),   D_i = dO_i . o_i
 *     dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i,
 * with Z redrawn from (seed, offset, p_drop) exactly as the forward call drew
 * it ("FlashAttention V2 核心原理与架构设计" §4.2, problem 3: forward and
 * backward must use one random pattern).  D_i = sum_j P_ij Z_ij (dO_i . v_j)
 * because o_i is the dropped output.  o and lse are those fa_fwd_dropout
 * wrote for the same q, k, v, causal, scale, p_drop, seed and offset.
 * Arguments, layouts and errors as fa_bwd; FA_ERR_INVALID_ARG also for
 * p_drop outside [0, 1) or NaN. */
fa_status fa_bwd_dropout(const void *q, const void *k, const void *v, const void *o,
                         const void *dO, const float *lse, float *ws, void *dq, void *dk,
                         void *dv, int B, int H, int N, int d, int causal, float scale,
                         float p_drop, unsigned long long seed, unsigned offset,
                         fa_dtype dtype, hipStream_t stream);

/* Backward pass of fa_fwd_window: the gradients fa_bwd computes, over the
 * allowed (query, key) pairs of fa_fwd_window's mask,
 *     max(0, i - window_left) <= j <= min(L_b - 1, i + window_right),
 * the sliding-window and padding masks of "FlashAttention 优化原理与实现要点解析"
 * §8 (reading as in fa_fwd.h).  Rows i >= L_b, which attend nothing, and
 * keys j >= L_b, which nothing attends, get zero gradients.
 *   o, lse          as fa_fwd_window wrote them for the same q, k, v, window,
 *                   seqlens and scale (rows i >= L_b: o = 0, lse = -inf)
 *   window_left, window_right, seqlens: as fa_fwd_window (sides >= -1, -1 =
 *                   open; seqlens device int32 [B] clamped to 0..N, or NULL)
 *   ws              fa_bwd_workspace_size(B, H, N) bytes, 16-byte aligned
 * Other arguments, layouts and errors as fa_bwd; FA_ERR_INVALID_ARG also for
 * a window side below -1 or seqlens overlapping an output, FA_ERR_MISALIGNED
 * for seqlens not 4-byte aligned.  seqlens is only read.  (-1, -1) without
 * seqlens gives fa_bwd's non-causal result and (-1, 0) its causal one. */
fa_status fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                        const void *dO, const float *lse, float *ws, void *dq, void *dk,
                        void *dv, int B, int H, int N, int d, int window_left,
                        int window_right, const int *seqlens, float scale, fa_dtype dtype,
                        hipStream_t stream);

/* Bytes of fp32 workspace fa_bwd_varlen needs (0 if a size is not
 * positive): per head, 32 * (ceil(total / 32) + B) rows of (lse, D). */
size_t fa_bwd_varlen_workspace_size(int B, int H, int total);

/* Backward pass of fa_fwd_varlen: within every packed sequence b (tokens
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head), the gradients fa_bwd
 * computes for that sequence alone, as if it were a [1,1,L_b,d] problem.
 *   q, k, v, o, dO  [H, total, d] 16-bit (o and lse as fa_fwd_varlen wrote
 *                   them for the same q, k, v, cu_seqlens, causal, scale),
 *                   read only
 *   lse             [H, total] fp32, read only
 *   cu_seqlens      device int32 [B + 1], the contract of fa_fwd_varlen
 *   ws              fa_bwd_varlen_workspace_size(B, H, total) bytes,
 *                   16-byte aligned, scratch
 *   dq, dk, dv      [H, total, d] 16-bit, written for every token inside a
 *                   sequence; rows of tokens outside every sequence
 *                   (cu_seqlens[B] .. total-1) are not written
 *   max_seqlen      the longest sequence (1 .. total); it sizes the grids
 * Bounds and lengths are clamped as in fa_fwd_varlen, so a malformed
 * cu_seqlens gives wrong rows, never an access outside the tensors or the
 * workspace.  Errors as fa_bwd, plus those fa_fwd_varlen adds for
 * cu_seqlens, total and max_seqlen.  Three kernels are enqueued on
 * `stream`; results are deterministic. */
fa_status fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                        const void *dO, const float *lse, const int *cu_seqlens, float *ws,
                        void *dq, void *dk, void *dv, int B, int H, int total,
                        int max_seqlen, int d, int causal, float scale, fa_dtype dtype,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
