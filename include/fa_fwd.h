/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) exact-attention forward pass.
 *
 * Operation.  For every batch b, head h and query row i,
 *     o[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:] . k[b,h,j,:]) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(scale * q[b,h,i,:] . k[b,h,j,:])
 * over the allowed keys j: all j < N, or j <= i when causal (square,
 * top-left aligned).  This is Attention(Q,K,V) = Softmax(Q K^T / sqrt(d)) V
 * of "FlashAttention 优化原理与实现要点解析" (cloud.baidu.com) §1, with the
 * caller's `scale` in place of 1/sqrt(d), and causal masking as in §7 of the
 * same page.  The N x N score matrix is never written to memory: Q-row tiles
 * stream K/V tiles through on-chip memory with a running maximum and sum
 * (§4.2-§6 of that page).  `lse` packs the two per-row statistics that the
 * kernel signature of "FlashAttention V2 核心原理与架构设计" (wmrh.cn) §2.3
 * returns separately (row maximum m and denominator l) into lse = m + ln l.
 *
 * Layout.  q, k, v and o are contiguous [B,H,N,d] arrays of one 16-bit type
 * (IEEE binary16 or bfloat16); element (b,h,n,c) is at ((b*H+h)*N+n)*d+c.
 * lse is a contiguous fp32 [B,H,N] array.  Accumulation is fp32; P is
 * rounded to the input type (nearest-even) before the P.V product, and o is
 * rounded to the input type (nearest-even) once, after the division by l.
 *
 * Ownership.  Every pointer is a device pointer owned by the caller; the
 * library allocates nothing and keeps no state between calls, so calls are
 * reentrant.  q, k and v are only read.  o and lse are fully overwritten
 * (all B*H*N rows) and must not overlap q, k, v or each other.
 *
 * Errors.  Arguments are validated on the host before any HIP call; a
 * failing call touches no memory and launches nothing.  A passing call
 * enqueues one kernel on `stream` (0 = the null stream) and returns without
 * waiting; device faults surface at the caller's next synchronisation.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,  /* null pointer, B/H/N < 1, causal not 0/1,
                                 non-finite scale, unknown dtype, overlapping
                                 buffers, or a grid too large to launch */
    FA_ERR_UNSUPPORTED = -2,  /* d not 64 or 128, or N above FA_MAX_N */
    FA_ERR_MISALIGNED = -3,   /* q, k, v or o not 16-byte aligned, lse not
                                 4-byte aligned */
    FA_ERR_LAUNCH = -4,       /* the kernel launch was rejected by HIP */
    FA_ERR_SCRATCH = -5       /* fa_fwd_split_noalloc: the partials need more
                                 than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

typedef enum { FA_DTYPE_F16 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/* Largest sequence length accepted: one head of K or V (N*d*2 bytes) must
 * stay addressable with 32-bit byte offsets. */
#define FA_MAX_N (1 << 22)

/* Forward pass on binary16 tensors.  Arguments as described above:
 *   q, k, v  [B,H,N,d] binary16, read only
 *   o        [B,H,N,d] binary16, written
 *   lse      [B,H,N]   fp32, written (natural log)
 *   B, H, N  batch, heads, sequence length (>= 1)
 *   d        head dimension, 64 or 128
 *   causal   0 = every key, 1 = keys j <= query i
 *   scale    finite multiplier of q.k (1/sqrt(d) in the usual definition);
 *            0 and negative values are accepted
 *   stream   HIP stream the kernel is enqueued on */
fa_status fa_fwd_f16(const void *q, const void *k, const void *v, void *o,
                     float *lse, int B, int H, int N, int d, int causal,
                     float scale, hipStream_t stream);

/* The same on bfloat16 tensors. */
fa_status fa_fwd_bf16(const void *q, const void *k, const void *v, void *o,
                      float *lse, int B, int H, int N, int d, int causal,
                      float scale, hipStream_t stream);

/* The same with the element type given explicitly. */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o,
                 float *lse, int B, int H, int N, int d, int causal,
                 float scale, fa_dtype dtype, hipStream_t stream);

/* Forward pass with a sliding window and per-batch valid lengths, the mask
 * kinds besides causal that "FlashAttention 优化原理与实现要点解析" §8 lists
 * (sliding-window and padding masks; the page defines neither, so):
 *   query i of batch element b attends key j when
 *       max(0, i - window_left) <= j <= min(L_b - 1, i + window_right)
 *   window_left, window_right >= 0, or -1 for no limit on that side
 *     (-1, -1) is fa_fwd non-causal and (-1, 0) is fa_fwd causal;
 *   seqlens: device int32 [B] of valid lengths L_b (values clamped to
 *     0..N), or NULL for L_b = N; keys j >= L_b are padding;
 *   rows i >= L_b attend nothing: o row = 0, lse = -inf.
 * Other arguments, layouts and errors as fa_fwd; also FA_ERR_INVALID_ARG for
 * a window side below -1 and FA_ERR_MISALIGNED for seqlens not 4-byte
 * aligned.  seqlens is only read. */
fa_status fa_fwd_window(const void *q, const void *k, const void *v, void *o,
                        float *lse, int B, int H, int N, int d, int window_left,
                        int window_right, const int *seqlens, float scale,
                        fa_dtype dtype, hipStream_t stream);

/* Forward pass over packed variable-length sequences, the padding mask kind
 * of "FlashAttention 优化原理与实现要点解析" §8 with the padding removed:
 * B sequences of different lengths are stored back to back along the token
 * axis and each attends only to itself.
 *   q, k, v, o   [H, total, d] 16-bit (element (h, t, c) at (h*total+t)*d+c)
 *   lse          [H, total] fp32
 *   cu_seqlens   device int32 [B + 1]: sequence b is tokens
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head; the caller
 *                guarantees 0 = cu_seqlens[0] <= cu_seqlens[1] <= ... <=
 *                cu_seqlens[B] <= total and every length <= max_seqlen
 *   max_seqlen   the longest sequence (1 .. total); it sizes the grid
 *   causal       0 = every key of the sequence, 1 = keys t' <= t within it
 *                (each sequence top-left aligned)
 * Within sequence b this is fa_fwd on its rows.  o and lse rows of tokens
 * outside every sequence (cu_seqlens[B] .. total-1) are not written.  The
 * kernel clamps the bounds it reads to [0, total] and each length to the
 * grid (ceil(max_seqlen / 256) 256-row blocks), so a malformed cu_seqlens
 * gives wrong rows, never an access outside the tensors.  Other arguments
 * and errors as fa_fwd: FA_ERR_INVALID_ARG also for a null cu_seqlens,
 * total < 1, max_seqlen outside 1 .. total, or cu_seqlens overlapping o or
 * lse; FA_ERR_UNSUPPORTED for max_seqlen > FA_MAX_N; FA_ERR_MISALIGNED for
 * cu_seqlens not 4-byte aligned.  cu_seqlens is only read. */
fa_status fa_fwd_varlen(const void *q, const void *k, const void *v, void *o,
                        float *lse, const int *cu_seqlens, int B, int H, int total,
                        int max_seqlen, int d, int causal, float scale, fa_dtype dtype,
                        hipStream_t stream);

/* Most key segments fa_fwd_split accepts. */
#define FA_MAX_SPLITS 64

/* Bytes of fp32 workspace fa_fwd_split needs (0 if an argument is invalid):
 * per non-empty key segment, a normalised fp32 O and an lse per row. */
size_t fa_fwd_split_workspace_size(int B, int H, int N, int d, int num_splits);

/* Forward pass with the keys of every row split into up to num_splits
 * segments (each a whole number of 128-key tiles) that separate
 * work-groups process, then merged per row with the same online-softmax
 * algebra the tiles use ("FlashAttention 优化原理与实现要点解析" §4.2-§4.3;
 * the split-K/V decoding of "FlashAttention V2 核心原理与架构设计" §5.1):
 *     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
 * It computes what fa_fwd computes; it pays off when B*H*ceil(N/256)
 * work-groups leave compute units idle (few heads, short-to-moderate N).
 *   num_splits  1 .. FA_MAX_SPLITS
 *   ws          fa_fwd_split_workspace_size bytes, 16-byte aligned, scratch
 * Other arguments and errors as fa_fwd (FA_ERR_INVALID_ARG also for
 * num_splits out of range, a null or overlapping ws; FA_ERR_MISALIGNED for
 * ws).  Two kernels are enqueued on `stream`. */
fa_status fa_fwd_split(const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int H, int N, int d, int causal,
                       float scale, int num_splits, float *ws, fa_dtype dtype,
                       hipStream_t stream);

/* Forward pass for decoding shapes: Nq query rows against Nk keys, the
 * long-sequence case that "FlashAttention V2 核心原理与架构设计" (wmrh.cn)
 * §5.1 hands to FlashDecoding (beyond 32K keys), computed as fa_fwd_split
 * computes it: the keys are cut into segments of whole 128-key tiles that
 * separate work-groups process, and a second kernel merges each row's
 * segment results (lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s).
 *     o[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:] . k[b,h,j,:]) v[b,h,j,:]
 * over the allowed keys: all j < Nk, or, when causal, j <= i + Nk - Nq --
 * the queries are the last Nq positions of the sequence (bottom-right
 * alignment; Nq = Nk is fa_fwd's square causal mask).  The page fixes no
 * shapes; this reading is the library's.
 *   q, o        contiguous [B,H,Nq,d], one 16-bit type
 *   k, v        contiguous [B,H,Nk,d], the same type
 *   lse         contiguous fp32 [B,H,Nq]
 *   Nq, Nk      1 .. FA_MAX_N; causal requires Nq <= Nk
 *   num_splits  0 (let the library choose: fa_fwd_decode_splits) or
 *               1 .. FA_MAX_SPLITS segments requested
 *   ws          fa_fwd_decode_workspace_size(B, H, Nq, Nk, d, num_splits)
 *               bytes of device scratch, 16-byte aligned
 * Other arguments, ownership and errors as fa_fwd: FA_ERR_INVALID_ARG also
 * for Nq > Nk when causal, num_splits out of range, a null ws or overlapping
 * buffers; FA_ERR_UNSUPPORTED for Nq or Nk above FA_MAX_N; FA_ERR_MISALIGNED
 * also for ws.  Two kernels are enqueued on `stream`. */
fa_status fa_fwd_decode(const void *q, const void *k, const void *v, void *o,
                        float *lse, int B, int H, int Nq, int Nk, int d,
                        int causal, float scale, int num_splits, float *ws,
                        fa_dtype dtype, hipStream_t stream);

/* Bytes of ws that fa_fwd_decode needs: segments x B*H*Nq x (d + 1) fp32,
 * where for Nq <= 32 every key segment counts twice (two waves of its
 * work-group each compute half of the segment's keys and leave their own
 * partial result).  0 for arguments fa_fwd_decode would reject as sizes. */
size_t fa_fwd_decode_workspace_size(int B, int H, int Nq, int Nk, int d,
                                    int num_splits);

/* The segment count fa_fwd_decode uses for num_splits = 0: about 256
 * work-groups over the grid (one per compute unit), with at least 4 tiles of
 * 128 keys per segment, at most FA_MAX_SPLITS.  0 for sizes below 1. */
int fa_fwd_decode_splits(int B, int H, int Nq, int Nk);

/* Size of the static per-device scratch of fa_fwd_split_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* fa_fwd_split for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, and harnesses that forbid
 * hipMalloc.  It takes no workspace argument and calls no allocator.  The
 * split partials go to a file-scope device array of FA_NOALLOC_SCRATCH_BYTES
 * bytes instead, which every device the library runs on holds from its first
 * call on that device (whose address the library looks up then) until the
 * process ends.  Results are bit-identical to fa_fwd_split with the same
 * arguments.
 *   stream  must belong to the current device (0 = its null stream)
 * Errors: as fa_fwd_split, and FA_ERR_SCRATCH (nothing launched) when
 * fa_fwd_split_workspace_size(B, H, N, d, num_splits) exceeds
 * FA_NOALLOC_SCRATCH_BYTES; FA_ERR_INVALID_ARG for a stream of another
 * device; FA_ERR_LAUNCH if HIP cannot report the current device, the stream's
 * device or the scratch address.  Every call on one device shares that
 * device's array, and the kernels overwrite every entry they later read, so
 * calls ordered on one stream need no clearing in between; calls that can
 * overlap on one device (different streams, no ordering) race on it. */
fa_status fa_fwd_split_noalloc(const void *q, const void *k, const void *v,
                               void *o, float *lse, int B, int H, int N, int d,
                               int causal, float scale, int num_splits,
                               fa_dtype dtype, hipStream_t stream);

/* Forward pass with dropout on the attention weights, the operation that
 * "FlashAttention V2 核心原理与架构设计" (wmrh.cn) fuses into the kernel
 * (§1.2, with a dropout_p argument in §5.2) and whose random pattern must be
 * the same in the forward and the backward pass (§4.2, problem 3).  The page
 * fixes no generator, mapping or scaling; this library uses:
 *     T    = floor((1 - p_drop) * 256 + 0.5), computed in double from the
 *            float p_drop
 *     keep element (b,h,i,j) iff byte 4*((j%32)/8) + j%4 (little-endian
 *            across the four output words) of Philox4x32-10 (Salmon et al.,
 *            SC 2011) with
 *              counter = (i, 2*(j/32) + (j/4)%2, b*H + h, offset)
 *              key     = (seed & 0xffffffff, seed >> 32)
 *            is below T
 *     o[b,h,i,:] = sum_j P_ij * Z_ij * v[b,h,j,:],  Z_ij = 256/T if kept,
 *            else 0 (every Z = 0 when T = 0)
 *     lse   unchanged: that of the undropped weights P.
 * A call with the same seed and offset draws the same pattern (the same
 * bits, on any stream or grid); fa_bwd_dropout redraws it.  Advancing the
 * offset (or the seed) between training steps gives fresh patterns.
 *   causal   0 or 1, as fa_fwd
 *   p_drop   dropout probability, 0 <= p_drop < 1 (p_drop = 0 keeps all)
 * Other arguments, layouts and errors as fa_fwd; FA_ERR_INVALID_ARG also for
 * p_drop outside [0, 1) or NaN. */
fa_status fa_fwd_dropout(const void *q, const void *k, const void *v, void *o,
                         float *lse, int B, int H, int N, int d, int causal,
                         float scale, float p_drop, unsigned long long seed,
                         unsigned offset, fa_dtype dtype, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char *fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
