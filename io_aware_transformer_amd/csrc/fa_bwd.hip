// fa_bwd.hip -- exact attention backward pass for MI355X (gfx950, CDNA4).
//
// Pages cited (by tag and section):
//   [P-notes] "FlashAttention v1 & v2 笔记"            (yiran529.github.io)
//   [P-baidu] "FlashAttention 优化原理与实现要点解析"    (cloud.baidu.com)
//   [P-wmrh]  "FlashAttention V2 核心原理与架构设计"     (wmrh.cn)
//
// The pages keep the forward pass's row statistics for the backward pass
// ([P-baidu] §6: numerator and denominator apart; [P-wmrh] §2.3 outputs l and
// m) but print no gradient formulas.  The gradients of
// O = Softmax(scale Q K^T) V for an upstream dO are, by the chain rule,
//   P = exp(scale Q K^T - lse)          recomputed per tile from the saved lse
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q
// and the N x N matrices P, dP, dS are never written to memory, as in the
// forward pass ([P-baidu] §4-§6 tiling).
//
// Three kernels, no atomics, so results are deterministic:
//  * delta: per row, lse * log2(e) and D = dO . O into a blocked fp32
//    workspace (per 32-row block: 32 values of lse*log2(e), then 32 of D;
//    rows past N get +inf and 0, so they contribute P = 0).
//  * dK/dV: one work-group per (batch*head, 256 keys); each of its 8 waves
//    keeps 32 keys' K fragments and fp32 dK^T, dV^T accumulators in VGPRs
//    and walks all query tiles (64 queries, double buffered in LDS with their
//    workspace rows).  V of the work-group's keys sits in LDS.  Per 32
//    queries: S = Q K^T, dP' = dO V^T - D (D preloaded into the MFMA
//    accumulator), P = 2^(S c - lse log2 e), dS = P dP', then
//    dV^T += dO^T P and dK^T += Q^T dS (transposing LDS reads of Q and dO).
//  * dQ: one work-group per (batch*head, 256 queries), like the forward: Q
//    and dO fragments stay in VGPRs, K/V tiles (64 keys) stream through
//    LDS, and per 32 keys S^T = K Q^T, dP'^T = V dO^T - D, dS^T = P^T dP'^T,
//    dQ^T += K^T dS^T.
// Both walking kernels skip the causal tiles wholly above the diagonal
// ([P-baidu] §7) and mask only the diagonal step.  Rows and keys past N
// need no mask: their Q, K, V and dO read as zero from the buffer range
// check, so every term they add to a stored output is zero.
//
// Dropout (fa_bwd_dropout): the walking kernels take a DROP flag that
// redraws the forward pass's keep factors Z from the same Philox counters
// ([P-wmrh] §4.2: forward and backward must draw one pattern) and computes
// dV = (P o Z)^T dO and dS = P o (Z o dP - D).
//
// Tiles in LDS use one 16-byte-chunk XOR swizzle that is bank-conflict free
// both for ds_read_b128 of 16 rows at one logical chunk and for the 4-row x
// 64-byte footprint of ds_read_b64_tr_b16, since Q, dO (dK/dV kernel) and K
// (dQ kernel) are read both ways.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

#include "fa_bwd.h"

namespace {

typedef unsigned short u16;
typedef u16 u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#define LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr unsigned kRsrcWord3 = 0x00020000u;     // raw buffer, 32-bit data
constexpr int kWsRows = 32;                      // rows per workspace block
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysA = 32 * kWaves;              // keys per dK/dV work-group
constexpr int kQT = 64;                          // queries per LDS tile (dK/dV)
constexpr int kQB = 32 * kWaves;                 // queries per dQ work-group
constexpr int kKT = 64;                          // keys per LDS tile (dQ)

template <int DT> struct Elem;

template <> struct Elem<FA_DTYPE_F16> {
    static __device__ __forceinline__ f32x16 mfma(u16x8 a, u16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f16x2 h = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(unsigned, h);
    }
    static __device__ __forceinline__ float lo(unsigned u) {
        return (float)__builtin_bit_cast(f16x2, u)[0];
    }
    static __device__ __forceinline__ float hi(unsigned u) {
        return (float)__builtin_bit_cast(f16x2, u)[1];
    }
};

template <> struct Elem<FA_DTYPE_BF16> {
    static __device__ __forceinline__ f32x16 mfma(u16x8 a, u16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        bf16x2 h = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(unsigned, h);
    }
    static __device__ __forceinline__ float lo(unsigned u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(unsigned u) {
        return __uint_as_float(u & 0xffff0000u);
    }
};

// Row geometry of a [rows, D] 16-bit tile in LDS and its chunk swizzle.
template <int D> struct Tile {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 1024 / kRowBytes; // rows per 1 KB load
    // d = 128 (16 chunks, 256-byte rows): chunk ^= (row&3)<<2 | (row>>2)&3,
    // a bijection on any 16 consecutive rows, and 4 consecutive rows (4-aligned)
    // get 4 different 64-byte chunk groups.  d = 64 (8 chunks, two rows per
    // 256 bytes): the same built from row>>1.
    static __device__ __forceinline__ int swz(int row) {
        return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                        : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
    }
};

template <int I> struct Buf { static constexpr int value = I; };

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kRsrcWord3);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds of two
// 32x32 -> 64-bit products (multipliers 0xD2511F53 on word 0, 0xCD9E8D57 on
// word 2), high halves XORed with the other words and the key, the key
// bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2,
                                               unsigned c3, unsigned k0, unsigned k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const unsigned long long a = (unsigned long long)0xD2511F53u * c0;
        const unsigned long long b = (unsigned long long)0xCD9E8D57u * c2;
        // three-input XORs (v_bitop3 truth table 0x96 = x ^ y ^ z)
        const unsigned n0 = __builtin_amdgcn_bitop3_b32((unsigned)(b >> 32), c1, k0, 0x96);
        const unsigned n2 = __builtin_amdgcn_bitop3_b32((unsigned)(a >> 32), c3, k1, 0x96);
        c1 = (unsigned)b;
        c3 = (unsigned)a;
        c0 = n0;
        c2 = n2;
    }
    const u32x4 r = {c0, c1, c2, c3};
    return r;
}

// Dropout parameters of one launch (as the forward pass): a weight is kept
// when its random byte is below thr; kept weights are scaled by fscale.
struct DropArgs {
    unsigned seed_lo, seed_hi, offset, thr;
    float fscale;
};

// Packed variable-length sequences (VARLEN kernels): tensors [H, total, d],
// sequence b of head h is rows cu[b] .. cu[b+1]-1 of the head (bounds
// clamped to [0, total], length to cap rows).  Its workspace rows start at
// 32 * (ceil(cu[b] / 32) + b) of the head's wsh rows, so sequences never
// share a 32-row workspace block.
struct VarlenArgs {
    const int *cu;
    int H, cap, wsh;
};

// This work-group's sequence: rows, first row in the [H*total, d] view,
// first workspace row.
struct Seq {
    int n;
    size_t row0, ws_row0;
};
__device__ __forceinline__ Seq varlen_seq(const VarlenArgs &vl, int bh, int total)
{
    const int b = bh / vl.H, h = bh % vl.H;
    const int start = min(max(vl.cu[b], 0), total);
    const int end = min(max(vl.cu[b + 1], start), total);
    Seq s;
    s.n = min(end - start, vl.cap);
    s.row0 = (size_t)h * (size_t)total + (size_t)start;
    s.ws_row0 = (size_t)h * (size_t)vl.wsh + 32 * ((size_t)((start + 31) / 32) + (size_t)b);
    return s;
}

// Sliding window and valid lengths (WIN kernels): query i of batch element
// b may attend key j when (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
// and both i and j are below the element's valid length L_b.
struct WindowArgs {
    const int *lens;   // device int32 [B] valid lengths (clamped to 0..N), or null
    int H, wl, wr;
};
__device__ __forceinline__ int window_len(const WindowArgs &wa, int bh, int N)
{
    return wa.lens ? min(max(wa.lens[bh / wa.H], 0), N) : N;
}
__device__ __forceinline__ bool window_allows(const WindowArgs &wa, int lb, int i, int j)
{
    return i < lb && j < lb && (wa.wl < 0 || j >= i - wa.wl) && (wa.wr < 0 || j <= i + wa.wr);
}

// Byte transpose of a 4x4 byte matrix held by the 4 lanes of a quad (lane e
// holds row e as one word): afterwards lane e holds column e.  Two stages:
// swap 16-bit halves with lane e^2, then bytes with lane e^1 (DPP quad
// permutes, v_perm_b32 with a per-lane selector).
struct QuadTranspose {
    unsigned sel1, sel2;
    __device__ __forceinline__ explicit QuadTranspose(int lane) {
        // v_perm_b32(a, b, sel): selector byte 0-3 takes a byte of b, 4-7 of a
        sel1 = (lane & 2) ? 0x07060302u : 0x01000504u;   // [y2 y3 x2 x3] : [x0 x1 y0 y1]
        sel2 = (lane & 1) ? 0x07030501u : 0x02060004u;   // [y1 x1 y3 x3] : [x0 y0 x2 y2]
    }
    __device__ __forceinline__ unsigned operator()(unsigned x) const {
        const unsigned y = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
        const unsigned z = __builtin_amdgcn_perm(x, y, sel1);
        const unsigned w = (unsigned)__builtin_amdgcn_mov_dpp((int)z, 0xB1, 0xF, 0xF, false);
        return __builtin_amdgcn_perm(z, w, sel2);
    }
};

// One 1 KB HBM -> LDS load of rows [row0, row0 + 1024 / (2 d)) of a swizzled
// [rows, d] tile: lane l lands at dst + 16 l, which is (row, physical chunk
// l % (d / 8)), so it fetches the logical chunk that belongs there.
__device__ __forceinline__ void load_rows(const __amdgpu_buffer_rsrc_t &r, LDS unsigned char *dst,
                                          int tile_row0, int src_row0, int lane, int d)
{
    const int chunks = d / 8;
    const int row = tile_row0 + lane / chunks;
    const int sw = d == 128 ? Tile<128>::swz(row) : Tile<64>::swz(row);
    const int lc = (lane % chunks) ^ sw;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (LDS void *)dst, 16, (src_row0 + lane / chunks) * 2 * d + lc * 16, 0, 0, 0);
}

// ---------------------------------------------------------------- delta

// ws block (bh, n / 32): [32 x lse*log2e][32 x -D]; rows n >= N get (+inf, 0).
// -D is stored because both gradient kernels start their dP' accumulators at
// -D: the dK/dV kernel loads it from LDS straight into the accumulator.
template <int DT, int D>
__global__ __launch_bounds__(256)
void fa_bwd_delta_kernel(const u16 *__restrict__ O, const u16 *__restrict__ dO,
                         const float *__restrict__ LSE, float *__restrict__ WS, int N,
                         int nblk, long long rows_padded)
{
    using E = Elem<DT>;
    constexpr int LPR = D / 8;                 // lanes per row, 8 elements each
    constexpr int RPB = 256 / LPR;
    const long long r = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    const long long bh = r / ((long long)nblk * kWsRows);
    const int n = (int)(r % ((long long)nblk * kWsRows));
    const bool valid = r < rows_padded && n < N;
    float acc = 0.f;
    if (valid) {
        const size_t off = ((size_t)bh * N + n) * D + part * 8;
        const u32x4 a = *(const u32x4 *)(O + off);
        const u32x4 b = *(const u32x4 *)(dO + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(E::lo(a[e]), E::lo(b[e]), acc);
            acc = fmaf(E::hi(a[e]), E::hi(b[e]), acc);
        }
    }
#pragma unroll
    for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    if (r < rows_padded && part == 0) {
        float *blk = WS + (size_t)(r / kWsRows) * (2 * kWsRows);
        const int i = (int)(r % kWsRows);
        blk[i] = valid ? LSE[(size_t)bh * N + n] * kLog2e : __builtin_inff();
        blk[kWsRows + i] = -acc;
    }
}

// The same for packed sequences: grid (row chunk, b*H + h); rows of the
// sequence's last 32-row workspace block past its length get (+inf, 0).
template <int DT, int D>
__global__ __launch_bounds__(256)
void fa_bwd_delta_varlen_kernel(const u16 *__restrict__ O, const u16 *__restrict__ dO,
                                const float *__restrict__ LSE, float *__restrict__ WS, int total,
                                VarlenArgs vl)
{
    using E = Elem<DT>;
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const Seq sq = varlen_seq(vl, blockIdx.y, total);
    const int r = blockIdx.x * RPB + threadIdx.x / LPR;    // row within the sequence
    const int part = threadIdx.x % LPR;
    const int padded = (sq.n + kWsRows - 1) / kWsRows * kWsRows;
    const bool valid = r < sq.n;
    float acc = 0.f;
    if (valid) {
        const size_t off = (sq.row0 + r) * D + part * 8;
        const u32x4 a = *(const u32x4 *)(O + off);
        const u32x4 b = *(const u32x4 *)(dO + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(E::lo(a[e]), E::lo(b[e]), acc);
            acc = fmaf(E::hi(a[e]), E::hi(b[e]), acc);
        }
    }
#pragma unroll
    for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    if (r < padded && part == 0) {
        const size_t idx = sq.ws_row0 + r;
        float *blk = WS + idx / kWsRows * (2 * kWsRows);
        const int i = (int)(idx % kWsRows);
        blk[i] = valid ? LSE[sq.row0 + r] * kLog2e : __builtin_inff();
        blk[kWsRows + i] = -acc;
    }
}

// ---------------------------------------------------------------- dK / dV

// DROP: the dropout of the forward pass, redrawn.  dV^T += dO^T (P o Z) and
// dS = P o (Z o dP - D).  A lane here holds one key and 16 queries, while a
// Philox call yields 16 keys of one query, so each lane makes the call of
// (query qs + l32, key half hh) of each step and the 32 x 32 bytes are
// transposed through a per-wave LDS block: a byte transpose inside each
// lane quad, 4 dword writes, and in the step one 16-byte read per lane.
template <int DT, int D, bool CAUSAL, bool DROP, bool VARLEN, bool WIN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(const u16 *__restrict__ Q, const u16 *__restrict__ K,
                        const u16 *__restrict__ V, const u16 *__restrict__ dO,
                        const float *__restrict__ WS, u16 *__restrict__ dK,
                        u16 *__restrict__ dV, int BH, int N_in, int nblk_in, float c2,
                        float scale, DropArgs dr, VarlenArgs vl, WindowArgs wa)
{
    static_assert(!(DROP && VARLEN), "dropout is built for the batched layout");
    static_assert(!(WIN && (CAUSAL || DROP || VARLEN)), "the window kernels stand alone");
    using E = Elem<DT>;
    using T = Tile<D>;
    constexpr int KT = D / 16;                 // MFMA k-steps over d
    constexpr int DB = D / 32;                 // 32-row blocks of dK^T, dV^T
    constexpr int QTB = kQT * T::kRowBytes;    // bytes of one Q or dO tile
    constexpr int TL = QTB / 1024;             // 1 KB loads per Q or dO tile
    static_assert(TL % kWaves == 0, "tile loads split evenly over the waves");

    // The per-step Q / dO tiles should sit in the first 64 KB, so that every
    // read of them is a lane offset plus an immediate (the reach of the
    // ds_read offset field); LDS objects are placed by decreasing alignment,
    // so the work-group's V rows (read at fixed addresses) get a smaller one.
    __shared__ __attribute__((aligned(1024))) unsigned char q0s[QTB];
    __shared__ __attribute__((aligned(1024))) unsigned char q1s[QTB];
    __shared__ __attribute__((aligned(1024))) unsigned char o0s[QTB];
    __shared__ __attribute__((aligned(1024))) unsigned char o1s[QTB];
    __shared__ __attribute__((aligned(256))) float w0s[2 * kQT];
    __shared__ __attribute__((aligned(256))) float w1s[2 * kQT];
    __shared__ __attribute__((aligned(512))) unsigned char vs[kKeysA * T::kRowBytes];
    // dropout bytes of one query tile, per wave: [step 2][key 32][query
    // half 2][g 4] words
    __shared__ __attribute__((aligned(1024))) unsigned zs[DROP ? kWaves * 512 : 1];
    auto qbuf = [&](auto b) -> LDS unsigned char * {
        if constexpr (decltype(b)::value == 0) return (LDS unsigned char *)q0s;
        else return (LDS unsigned char *)q1s;
    };
    auto obuf = [&](auto b) -> LDS unsigned char * {
        if constexpr (decltype(b)::value == 0) return (LDS unsigned char *)o0s;
        else return (LDS unsigned char *)o1s;
    };
    auto wbuf = [&](auto b) -> LDS float * {
        if constexpr (decltype(b)::value == 0) return (LDS float *)w0s;
        else return (LDS float *)w1s;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int L = blockIdx.x;
    const int bh = L % BH;
    const int kb = L / BH;                     // causal: low key blocks (most work) first
    // this work-group's problem: N rows starting at row0 of the [rows, d]
    // view, workspace blocks from ws_blk0 (nblk of them)
    int N = N_in, nblk = nblk_in;
    size_t row0 = (size_t)bh * (size_t)N_in, ws_blk0 = (size_t)bh * nblk_in;
    if constexpr (VARLEN) {
        const Seq sq = varlen_seq(vl, bh, N_in);
        N = sq.n;
        nblk = (N + kWsRows - 1) / kWsRows;
        row0 = sq.row0;
        ws_blk0 = sq.ws_row0 / kWsRows;
        if (kb * kKeysA >= N) return;          // key block past the sequence
    }
    const size_t head = row0 * D;
    const int nbytes = N * T::kRowBytes;
    const __amdgpu_buffer_rsrc_t rq = rsrc(Q + head, nbytes);
    const __amdgpu_buffer_rsrc_t rk = rsrc(K + head, nbytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc(V + head, nbytes);
    const __amdgpu_buffer_rsrc_t rdo = rsrc(dO + head, nbytes);
    const __amdgpu_buffer_rsrc_t rw = rsrc(WS + ws_blk0 * (2 * kWsRows), nblk * 2 * kWsRows * 4);

    const int k0 = kb * kKeysA;
    const int kw = k0 + 32 * w;                // this wave's first key
    const int key = kw + l32;                  // this lane's key (MFMA column)

    // K fragments: B operand of S = Q K^T (column = key, 8 consecutive d)
    u16x8 kf[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rk, (key * D + 16 * kk + 8 * hh) * 2, 0, 0);
        kf[kk] = __builtin_bit_cast(u16x8, x);
    }

    // V rows of the work-group's keys -> LDS, once
    constexpr int VL = kKeysA * T::kRowBytes / 1024 / kWaves;
#pragma unroll
    for (int j = 0; j < VL; ++j) {
        const int li = j * kWaves + w;
        load_rows(rv, (LDS unsigned char *)vs + li * 1024, li * T::kRowsPerLoad,
                     k0 + li * T::kRowsPerLoad, lane, D);
    }

    const int n_qt = (N + kQT - 1) / kQT;
    int t0 = CAUSAL ? k0 / kQT : 0, t_end = n_qt;
    // window: the query rows any key of this work-group may be attended by,
    // and this wave's (rows past lb and keys past lb take no part)
    int lb = N, wq_lo = 0, wq_hi = -1;
    if constexpr (WIN) {
        lb = window_len(wa, bh, N);
        const int k_last = min(k0 + kKeysA, lb) - 1;
        const int q_lo = wa.wr < 0 ? 0 : max(0, k0 - wa.wr);
        const int q_hi = wa.wl < 0 ? lb - 1 : min(lb - 1, k_last + wa.wl);
        t0 = t_end = 0;
        if (k0 < lb && q_lo <= q_hi) {
            t0 = q_lo / kQT;
            t_end = q_hi / kQT + 1;
        }
        if (kw < lb) {
            wq_lo = wa.wr < 0 ? 0 : kw - wa.wr;
            wq_hi = wa.wl < 0 ? lb - 1 : min(lb - 1, min(kw + 31, lb - 1) + wa.wl);
        }
    }
    const int ws_wave = __builtin_amdgcn_readfirstlane(w);

    auto issue = [&](auto par, int t) {
#pragma unroll
        for (int j = 0; j < TL / kWaves; ++j) {
            const int lt = j * kWaves + w;
            load_rows(rq, qbuf(par) + lt * 1024, lt * T::kRowsPerLoad,
                         t * kQT + lt * T::kRowsPerLoad, lane, D);
            load_rows(rdo, obuf(par) + lt * 1024, lt * T::kRowsPerLoad,
                         t * kQT + lt * T::kRowsPerLoad, lane, D);
        }
        if (ws_wave == kWaves - 1) {
#pragma unroll
            for (int j = 0; j < kQT / kWsRows; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (LDS void *)(wbuf(par) + j * 2 * kWsRows), 4,
                    ((t * (kQT / kWsRows) + j) * 2 * kWsRows + lane) * 4, 0, 0, 0);
        }
    };

    // per-lane LDS offsets (loop invariant)
    // Per-lane LDS offsets.  The row part of each offset is a multiple of 128
    // and the chunk part lies in bits 4-6 (d = 64) or 4-7 (d = 128), so a
    // compile-time chunk change is an XOR of the lane's base offset.
    // b128 row reads (row l32, logical chunk 2kk + hh): roff0 ^ (kk << 5)
    const int roff0 = l32 * T::kRowBytes + ((hh ^ T::swz(l32)) << 4);
    // transposing reads (rows 8h + 0..7 of a 16-row step, d block db):
    // toff0[h] ^ (db << 6)
    int toff0[2];
    {
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + 4 * (g >> 1) + (i >> 2);
            const int dl = 16 * (g & 1) + 4 * (i & 3);
            toff0[h] = row * T::kRowBytes + (((dl >> 3) ^ T::swz(row)) << 4) + ((dl >> 2) & 1) * 8;
        }
    }
    const int voff = 32 * w * T::kRowBytes;    // this wave's keys in vs

    auto rfrag = [&](LDS unsigned char *buf, int u, int kk) -> u16x8 {
        return *(const LDS u16x8 *)(buf + 32 * u * T::kRowBytes + (roff0 ^ (kk << 5)));
    };
    auto tfrag = [&](LDS unsigned char *buf, int u, int db, int ks) -> u16x8 {
        LDS unsigned char *p = buf + (32 * u + 16 * ks) * T::kRowBytes;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)(p + (toff0[0] ^ (db << 6))));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)(p + (toff0[1] ^ (db << 6))));
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dva[db][r] = dka[db][r] = 0.f;

    // Dropout bytes of step qs, as lane (key kw + l32, query half hh) needs
    // them: word g, byte e is query qs + 8g + 4hh + e (the accumulator row of
    // register 4g + e).  Lane (query m = l32, key half hh) draws the call for
    // query qs + m; its word gk, byte ek is key 8gk + 4hh + ek.  After the
    // quad transpose, word gk of lane (quad a = m/4, position e = m%4) holds,
    // for key 8gk + 4hh + e, the four queries 4a..4a+3: word a/2 of query
    // half a%2.
    // The bytes of a whole query tile are drawn before its steps, while only
    // the K fragments and the accumulators are live, so no Philox state
    // shares the registers with S and dP; a step reads its 16 bytes back
    // with one ds_read_b128.
    LDS unsigned *zw = (LDS unsigned *)zs + (DROP ? 512 * w : 0);
    auto drop_tile = [&](int t) {
        const QuadTranspose qtr(lane);
        const int a = l32 >> 2, e = l32 & 3;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int u = 0; u < kQT / 32; ++u) {
            const int qs = t * kQT + 32 * u;
            if ((CAUSAL && qs + 31 < kw) || qs >= N) continue;   // step not computed
            const u32x4 r = philox4x32_10((unsigned)(qs + l32), (unsigned)(2 * (kw / 32) + hh),
                                          (unsigned)bh, dr.offset, dr.seed_lo, dr.seed_hi);
#pragma unroll
            for (int gk = 0; gk < 4; ++gk)
                zw[256 * u + (8 * gk + 4 * hh + e) * 8 + (a & 1) * 4 + (a >> 1)] = qtr(r[gk]);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    auto drop_bytes = [&](int u) -> u32x4 {
        return *(const LDS u32x4 *)(zw + 256 * u + l32 * 8 + hh * 4);
    };

    // one step: 32 queries (sub-step u of the tile in buffers par).  Every
    // MFMA loop reads its LDS operands a fixed distance ahead, and the
    // interleave is pinned (scheduling-group barriers) so that neither the
    // reads crowd the registers nor each MFMA waits on its own read.
    auto step = [&](auto par, int u, bool diag, int qs) {
        LDS unsigned char *qb = qbuf(par);
        LDS unsigned char *ob = obuf(par);
        LDS float *wb = wbuf(par) + u * 2 * kWsRows;
        // S = Q K^T
        f32x16 s = {};
        {
            constexpr int AH = 2;
            u16x8 a[KT];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < AH; ++i) a[i] = rfrag(qb, u, i);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                if (kk + AH < KT) a[kk + AH] = rfrag(qb, u, kk + AH);
                s = E::mfma(a[kk], kf[kk], s);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
            for (int i = 0; i < KT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < KT - AH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // dP' = dO V^T - D: the accumulator starts at -D of the lane's rows,
        // as stored (at 0 under dropout, where D enters after the keep factor)
        f32x16 dp;
        if constexpr (DROP) {
            dp = f32x16{};
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 nd4 = *(const LDS f32x4 *)(wb + kWsRows + 8 * g + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd4[e];
            }
        }
        {
            // one MFMA ahead at d = 128: two ahead overflows the 256 VGPRs
            // there (K fragments, dK/dV accumulators, S and dP are live)
            constexpr int AH = D == 128 ? 1 : 2;
            u16x8 a[KT], bv[KT];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < AH; ++i) {
                a[i] = rfrag(ob, u, i);
                bv[i] = *(const LDS u16x8 *)((LDS unsigned char *)vs + voff + (roff0 ^ (i << 5)));
            }
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                if (kk + AH < KT) {
                    a[kk + AH] = rfrag(ob, u, kk + AH);
                    bv[kk + AH] = *(const LDS u16x8 *)((LDS unsigned char *)vs + voff +
                                                       (roff0 ^ ((kk + AH) << 5)));
                }
                dp = E::mfma(a[kk], bv[kk], dp);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH + 4, 0);
#pragma unroll
            for (int i = 0; i < KT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < KT - AH) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // P = 2^(S c2 - lse log2 e), dS = P dP'; rows m = 8(r/4) + 4hh + r%4
        u32x4 zb;
        if constexpr (DROP) zb = drop_bytes(u);
        u32x4 pp[2], dsp[2];
        float xv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *(const LDS f32x4 *)(wb + 8 * g + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * g + e] = fmaf(s[4 * g + e], c2, -l4[e]);
        }
        // the mask only on masked steps: a branch on the wave-uniform flag,
        // so that the other steps carry none of its selects
        if (__builtin_amdgcn_readfirstlane((int)diag)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 8 * (r >> 2) + 4 * hh + (r & 3);   // query qs + m
                bool masked;
                if constexpr (WIN) masked = !window_allows(wa, lb, qs + m, kw + l32);
                else masked = l32 > m;
                if (masked) xv[r] = neg_inf();
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 nd4;   // -D of the four rows
            if constexpr (DROP) nd4 = *(const LDS f32x4 *)(wb + kWsRows + 8 * g + 4 * hh);
            float p[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = __builtin_amdgcn_exp2f(xv[4 * g + e]);
                if constexpr (DROP) {
                    // dS = P (Z dP - D), and P Z for the dV product
                    const float zf = ((zb[g] >> (8 * e)) & 0xffu) < dr.thr ? dr.fscale : 0.f;
                    ds[e] = p[e] * fmaf(zf, dp[4 * g + e], nd4[e]);
                    p[e] *= zf;
                } else {
                    ds[e] = p[e] * dp[4 * g + e];
                }
            }
            pp[g >> 1][2 * (g & 1)] = E::pack2(p[0], p[1]);
            pp[g >> 1][2 * (g & 1) + 1] = E::pack2(p[2], p[3]);
            dsp[g >> 1][2 * (g & 1)] = E::pack2(ds[0], ds[1]);
            dsp[g >> 1][2 * (g & 1) + 1] = E::pack2(ds[2], ds[3]);
        }
        // dV^T += dO^T P,  dK^T += Q^T dS  (k-steps of 16 queries)
        {
            constexpr int NM = 2 * DB;          // (ks, db) pairs, each one dV and one dK MFMA
            constexpr int AH = 2;
            u16x8 ta[NM], tb[NM];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < AH; ++i) {
                ta[i] = tfrag(ob, u, i % DB, i / DB);
                tb[i] = tfrag(qb, u, i % DB, i / DB);
            }
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + AH < NM) {
                    ta[i + AH] = tfrag(ob, u, (i + AH) % DB, (i + AH) / DB);
                    tb[i + AH] = tfrag(qb, u, (i + AH) % DB, (i + AH) / DB);
                }
                const int db = i % DB, ks = i / DB;
                dva[db] = E::mfma(ta[i], __builtin_bit_cast(u16x8, pp[ks]), dva[db]);
                dka[db] = E::mfma(tb[i], __builtin_bit_cast(u16x8, dsp[ks]), dka[db]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * AH, 0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (i < NM - AH) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto tile = [&](auto par, int t) {
        constexpr int P = decltype(par)::value;
        if (t + 1 < t_end) issue(Buf<1 - P>{}, t + 1);
        if constexpr (DROP) drop_tile(t);
#pragma unroll
        for (int u = 0; u < kQT / 32; ++u) {
            const int qs = t * kQT + 32 * u;   // first query of the step
            // under dropout a step wholly past N (which adds nothing) is
            // skipped too: the branch keeps the register allocator from
            // spilling across the fused steps of the non-causal kernel
            if constexpr (WIN) {
                // some pair of the step allowed; a mask unless all are
                if (qs <= wq_hi && qs + 31 >= wq_lo) {
                    const bool all = (wa.wr < 0 || kw + 31 <= qs + wa.wr) &&
                                     (wa.wl < 0 || kw >= qs + 31 - wa.wl) &&
                                     kw + 31 < lb && qs + 31 < lb;
                    step(par, u, !all, qs);
                }
            } else if ((!CAUSAL || qs + 31 >= kw) && (!DROP || qs < N)) {
                step(par, u, CAUSAL && qs == kw, qs);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (t0 < t_end) issue(Buf<0>{}, t0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = t0; t < t_end; t += 2) {
        tile(Buf<0>{}, t);
        if (t + 1 < t_end) tile(Buf<1>{}, t + 1);
    }

    // epilogue: dK = scale dK^T, dV = dV^T, rows of key `key`, d = 32db + 8g + 4hh + e
    if (key < N) {
        u16 *dkr = dK + head + (size_t)key * D;
        u16 *dvr = dV + head + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 a, b;
                a[0] = E::pack2(dka[db][4 * g] * scale, dka[db][4 * g + 1] * scale);
                a[1] = E::pack2(dka[db][4 * g + 2] * scale, dka[db][4 * g + 3] * scale);
                b[0] = E::pack2(dva[db][4 * g], dva[db][4 * g + 1]);
                b[1] = E::pack2(dva[db][4 * g + 2], dva[db][4 * g + 3]);
                *(u32x2 *)(dkr + 32 * db + 8 * g + 4 * hh) = a;
                *(u32x2 *)(dvr + 32 * db + 8 * g + 4 * hh) = b;
            }
    }
}

// ---------------------------------------------------------------- dQ

// DROP: dS = P o (Z o dP - D) with the forward's keep factors Z; a lane
// holds 16 keys of one query, the 16 bytes of one Philox call per step.
template <int DT, int D, bool CAUSAL, bool DROP, bool VARLEN, bool WIN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(const u16 *__restrict__ Q, const u16 *__restrict__ K,
                      const u16 *__restrict__ V, const u16 *__restrict__ dO,
                      const float *__restrict__ WS, u16 *__restrict__ dQ, int BH, int N_in,
                      int nblk, int nqb, float c2, float scale, DropArgs dr, VarlenArgs vl,
                      WindowArgs wa)
{
    static_assert(!(DROP && VARLEN), "dropout is built for the batched layout");
    static_assert(!(WIN && (CAUSAL || DROP || VARLEN)), "the window kernels stand alone");
    using E = Elem<DT>;
    using T = Tile<D>;
    constexpr int KT = D / 16;
    constexpr int DB = D / 32;
    constexpr int KTB = kKT * T::kRowBytes;    // bytes of one K or V tile
    constexpr int TL = KTB / 1024;
    static_assert(TL % kWaves == 0, "tile loads split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) unsigned char k0s[KTB];
    __shared__ __attribute__((aligned(1024))) unsigned char k1s[KTB];
    __shared__ __attribute__((aligned(1024))) unsigned char v0s[KTB];
    __shared__ __attribute__((aligned(1024))) unsigned char v1s[KTB];
    auto kbuf = [&](auto b) -> LDS unsigned char * {
        if constexpr (decltype(b)::value == 0) return (LDS unsigned char *)k0s;
        else return (LDS unsigned char *)k1s;
    };
    auto vbuf = [&](auto b) -> LDS unsigned char * {
        if constexpr (decltype(b)::value == 0) return (LDS unsigned char *)v0s;
        else return (LDS unsigned char *)v1s;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int L = blockIdx.x;
    const int bh = L % BH;
    const int qblk = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
    int N = N_in;
    size_t row0 = (size_t)bh * (size_t)N_in, ws_blk0 = (size_t)bh * nblk;
    if constexpr (VARLEN) {
        const Seq sq = varlen_seq(vl, bh, N_in);
        N = sq.n;
        row0 = sq.row0;
        ws_blk0 = sq.ws_row0 / kWsRows;
        if (qblk * kQB >= N) return;           // Q block past the sequence
    }
    const size_t head = row0 * D;
    const int nbytes = N * T::kRowBytes;
    const __amdgpu_buffer_rsrc_t rq = rsrc(Q + head, nbytes);
    const __amdgpu_buffer_rsrc_t rk = rsrc(K + head, nbytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc(V + head, nbytes);
    const __amdgpu_buffer_rsrc_t rdo = rsrc(dO + head, nbytes);

    const int q0 = qblk * kQB + 32 * w;        // this wave's first query
    const int qrow = q0 + l32;                 // this lane's query (MFMA column)

    // Q and dO fragments: B operands (column = query, 8 consecutive d)
    u16x8 qf[KT], of[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        const int off = (qrow * D + 16 * kk + 8 * hh) * 2;
        qf[kk] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        of[kk] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
    }
    // this lane's row statistics (rows past N read as +inf and 0)
    float l2 = __builtin_inff(), nd = 0.f;   // lse log2(e) and -D of the row
    if (qrow < N) {
        const float *blk = WS + (ws_blk0 + qrow / kWsRows) * (2 * kWsRows);
        l2 = blk[qrow % kWsRows];
        nd = blk[kWsRows + qrow % kWsRows];
    }

    const int n_kt32 = (N + 31) / 32;
    const int n_steps = CAUSAL ? min(n_kt32, (qblk + 1) * (kQB / 32)) : n_kt32;
    int t_begin = 0, t_end = (n_steps + 1) / 2;
    const int n_w = (q0 >= N) ? 0 : (CAUSAL ? min(n_steps, q0 / 32 + 1) : n_steps);
    // window: the keys any row of this work-group may attend, and this
    // wave's (rows past lb and keys past lb take no part)
    int lb = N, wk_lo = 0, wk_hi = -1;
    if constexpr (WIN) {
        lb = window_len(wa, bh, N);
        const int qb0 = qblk * kQB;
        const int q_last = min(qb0 + kQB, lb) - 1;
        const int k_lo = wa.wl < 0 ? 0 : max(0, qb0 - wa.wl);
        const int k_hi = wa.wr < 0 ? lb - 1 : min(lb - 1, q_last + wa.wr);
        t_begin = t_end = 0;
        if (qb0 < lb && k_lo <= k_hi) {
            t_begin = k_lo / kKT;
            t_end = k_hi / kKT + 1;
        }
        if (q0 < lb) {
            wk_lo = wa.wl < 0 ? 0 : q0 - wa.wl;
            wk_hi = wa.wr < 0 ? lb - 1 : min(lb - 1, min(q0 + 31, lb - 1) + wa.wr);
        }
    }

    auto issue = [&](auto par, int t) {
#pragma unroll
        for (int j = 0; j < TL / kWaves; ++j) {
            const int lt = j * kWaves + w;
            load_rows(rk, kbuf(par) + lt * 1024, lt * T::kRowsPerLoad,
                         t * kKT + lt * T::kRowsPerLoad, lane, D);
            load_rows(rv, vbuf(par) + lt * 1024, lt * T::kRowsPerLoad,
                         t * kKT + lt * T::kRowsPerLoad, lane, D);
        }
    };

    // Per-lane LDS offsets.  The row part of each offset is a multiple of 128
    // and the chunk part lies in bits 4-6 (d = 64) or 4-7 (d = 128), so a
    // compile-time chunk change is an XOR of the lane's base offset.
    // b128 row reads (row l32, logical chunk 2kk + hh): roff0 ^ (kk << 5)
    const int roff0 = l32 * T::kRowBytes + ((hh ^ T::swz(l32)) << 4);
    // transposing reads (rows 8h + 0..7 of a 16-row step, d block db):
    // toff0[h] ^ (db << 6)
    int toff0[2];
    {
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + 4 * (g >> 1) + (i >> 2);
            const int dl = 16 * (g & 1) + 4 * (i & 3);
            toff0[h] = row * T::kRowBytes + (((dl >> 3) ^ T::swz(row)) << 4) + ((dl >> 2) & 1) * 8;
        }
    }
    auto rfrag = [&](LDS unsigned char *buf, int u, int kk) -> u16x8 {
        return *(const LDS u16x8 *)(buf + 32 * u * T::kRowBytes + (roff0 ^ (kk << 5)));
    };
    auto tfrag = [&](LDS unsigned char *buf, int u, int db, int ks) -> u16x8 {
        LDS unsigned char *p = buf + (32 * u + 16 * ks) * T::kRowBytes;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)(p + (toff0[0] ^ (db << 6))));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)(p + (toff0[1] ^ (db << 6))));
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 dqa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

    // one step: 32 keys (sub-step u of the tile in buffers par)
    auto step = [&](auto par, int u, bool diag, int ks0) {
        LDS unsigned char *kb = kbuf(par);
        LDS unsigned char *vb = vbuf(par);
        // S^T and dP'^T as two interleaved MFMA chains; operand i (K for even
        // i, V for odd) read from LDS AH MFMAs ahead, the interleave pinned
        f32x16 s = {}, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = DROP ? 0.f : nd;
        {
            constexpr int NR = 2 * KT;
            constexpr int AH = 3;
            u16x8 a[NR];
            auto frag = [&](int i) -> u16x8 {
                return (i & 1) ? rfrag(vb, u, i >> 1) : rfrag(kb, u, i >> 1);
            };
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < AH; ++i) a[i] = frag(i);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                if (i + AH < NR) a[i + AH] = frag(i + AH);
                if (i & 1) dp = E::mfma(a[i], of[i >> 1], dp);
                else s = E::mfma(a[i], qf[i >> 1], s);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NR - AH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // rows = keys ks0 + 8(r/4) + 4hh + r%4, column = query qrow; under
        // dropout register 4g + e is byte 4g + e of the step's call
        u32x4 zb;
        if constexpr (DROP)
            zb = philox4x32_10((unsigned)qrow, (unsigned)(2 * (ks0 / 32) + hh), (unsigned)bh,
                               dr.offset, dr.seed_lo, dr.seed_hi);
        u32x4 dsp[2];
        float xv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[r] = fmaf(s[r], c2, -l2);
        // the mask only on masked steps: a branch on the wave-uniform flag,
        // so that the other steps carry none of its compares and selects
        if (__builtin_amdgcn_readfirstlane((int)diag)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = ks0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                bool masked;
                if constexpr (WIN) masked = !window_allows(wa, lb, qrow, key);
                else masked = key > qrow;
                if (masked) xv[r] = neg_inf();
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = xv[4 * g + e];
                if constexpr (DROP) {
                    const float zf = ((zb[g] >> (8 * e)) & 0xffu) < dr.thr ? dr.fscale : 0.f;
                    ds[e] = __builtin_amdgcn_exp2f(x) * fmaf(zf, dp[4 * g + e], nd);
                } else {
                    ds[e] = __builtin_amdgcn_exp2f(x) * dp[4 * g + e];
                }
            }
            dsp[g >> 1][2 * (g & 1)] = E::pack2(ds[0], ds[1]);
            dsp[g >> 1][2 * (g & 1) + 1] = E::pack2(ds[2], ds[3]);
        }
        // dQ^T += K^T dS^T, transposing reads of K two per MFMA, AH ahead
        {
            constexpr int NM = 2 * DB;
            constexpr int AH = 2;
            u16x8 tk[NM];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < AH; ++i) tk[i] = tfrag(kb, u, i % DB, i / DB);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + AH < NM) tk[i + AH] = tfrag(kb, u, (i + AH) % DB, (i + AH) / DB);
                dqa[i % DB] = E::mfma(tk[i], __builtin_bit_cast(u16x8, dsp[i / DB]), dqa[i % DB]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NM - AH) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto tile = [&](auto par, int t) {
        constexpr int P = decltype(par)::value;
        if (t + 1 < t_end) issue(Buf<1 - P>{}, t + 1);
#pragma unroll
        for (int u = 0; u < kKT / 32; ++u) {
            const int j = t * (kKT / 32) + u;  // 32-key step index
            if constexpr (WIN) {
                const int ks = 32 * j;
                if (ks <= wk_hi && ks + 31 >= wk_lo) {
                    const bool all = (wa.wl < 0 || ks >= q0 + 31 - wa.wl) &&
                                     (wa.wr < 0 || ks + 31 <= q0 + wa.wr) &&
                                     ks + 31 < lb && q0 + 31 < lb;
                    step(par, u, !all, ks);
                }
            } else if (j < n_w) {
                step(par, u, CAUSAL && 32 * j + 31 > q0, 32 * j);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (t_begin < t_end) issue(Buf<0>{}, t_begin);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = t_begin; t < t_end; t += 2) {
        tile(Buf<0>{}, t);
        if (t + 1 < t_end) tile(Buf<1>{}, t + 1);
    }

    if (qrow < N) {
        u16 *r = dQ + head + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 a;
                a[0] = E::pack2(dqa[db][4 * g] * scale, dqa[db][4 * g + 1] * scale);
                a[1] = E::pack2(dqa[db][4 * g + 2] * scale, dqa[db][4 * g + 3] * scale);
                *(u32x2 *)(r + 32 * db + 8 * g + 4 * hh) = a;
            }
    }
}

// ---------------------------------------------------------------- host

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

template <int DT, int D, bool CAUSAL, bool DROP>
hipError_t launch(const void *q, const void *k, const void *v, const void *o, const void *dO,
                  const float *lse, float *ws, void *dq, void *dk, void *dv, int BH, int N,
                  float scale, DropArgs dr, hipStream_t stream)
{
    const VarlenArgs vl = {nullptr, 1, 0, 0};
    const WindowArgs wa = {nullptr, 1, -1, -1};
    const int nblk = (N + kWsRows - 1) / kWsRows;
    const long long rows_padded = (long long)BH * nblk * kWsRows;
    constexpr int RPB = 256 / (D / 8);
    const long long g1 = (rows_padded + RPB - 1) / RPB;
    const int nkb = (N + kKeysA - 1) / kKeysA;
    const int nqb = (N + kQB - 1) / kQB;
    const float c2 = scale * kLog2e;
    hipLaunchKernelGGL((fa_bwd_delta_kernel<DT, D>), dim3((unsigned)g1), dim3(256), 0, stream,
                       (const u16 *)o, (const u16 *)dO, lse, ws, N, nblk, rows_padded);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DT, D, CAUSAL, DROP, false>),
                       dim3((unsigned)((long long)BH * nkb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dk, (u16 *)dv, BH, N, nblk, c2, scale, dr, vl, wa);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DT, D, CAUSAL, DROP, false>),
                       dim3((unsigned)((long long)BH * nqb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dq, BH, N, nblk, nqb, c2, scale, dr, vl, wa);
    return hipGetLastError();
}

// Packed sequences: total rows per head, at most cap (a multiple of 256)
// rows per sequence.
template <int DT, int D, bool CAUSAL>
hipError_t launch_varlen(const void *q, const void *k, const void *v, const void *o,
                         const void *dO, const float *lse, float *ws, void *dq, void *dk,
                         void *dv, int BH, int total, VarlenArgs vl, float scale,
                         hipStream_t stream)
{
    constexpr int RPB = 256 / (D / 8);
    const DropArgs dr = {0u, 0u, 0u, 256u, 1.f};
    const WindowArgs wa = {nullptr, 1, -1, -1};
    const float c2 = scale * kLog2e;
    const int nb = vl.cap / kKeysA;            // key blocks = Q blocks per sequence
    hipLaunchKernelGGL((fa_bwd_delta_varlen_kernel<DT, D>),
                       dim3((unsigned)((vl.cap + RPB - 1) / RPB), (unsigned)BH), dim3(256), 0,
                       stream, (const u16 *)o, (const u16 *)dO, lse, ws, total, vl);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DT, D, CAUSAL, false, true>),
                       dim3((unsigned)((long long)BH * nb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dk, (u16 *)dv, BH, total, 0, c2, scale, dr, vl, wa);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DT, D, CAUSAL, false, true>),
                       dim3((unsigned)((long long)BH * nb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dq, BH, total, 0, nb, c2, scale, dr, vl, wa);
    return hipGetLastError();
}

typedef hipError_t (*launch_varlen_fn)(const void *, const void *, const void *, const void *,
                                       const void *, const float *, float *, void *, void *,
                                       void *, int, int, VarlenArgs, float, hipStream_t);

template <int DT>
launch_varlen_fn pick_varlen(int d, int causal)
{
    if (d == 64) return causal ? launch_varlen<DT, 64, true> : launch_varlen<DT, 64, false>;
    return causal ? launch_varlen<DT, 128, true> : launch_varlen<DT, 128, false>;
}

// Window and valid lengths: the batched row-term kernel, then the WIN walking
// kernels over the full [B,H,N,d] grid.
template <int DT, int D>
hipError_t launch_window(const void *q, const void *k, const void *v, const void *o,
                         const void *dO, const float *lse, float *ws, void *dq, void *dk,
                         void *dv, int BH, int N, WindowArgs wa, float scale, hipStream_t stream)
{
    const VarlenArgs vl = {nullptr, 1, 0, 0};
    const DropArgs dr = {0u, 0u, 0u, 256u, 1.f};
    const int nblk = (N + kWsRows - 1) / kWsRows;
    const long long rows_padded = (long long)BH * nblk * kWsRows;
    constexpr int RPB = 256 / (D / 8);
    const long long g1 = (rows_padded + RPB - 1) / RPB;
    const float c2 = scale * kLog2e;
    hipLaunchKernelGGL((fa_bwd_delta_kernel<DT, D>), dim3((unsigned)g1), dim3(256), 0, stream,
                       (const u16 *)o, (const u16 *)dO, lse, ws, N, nblk, rows_padded);
    const int nkb = (N + kKeysA - 1) / kKeysA;
    const int nqb = (N + kQB - 1) / kQB;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DT, D, false, false, false, true>),
                       dim3((unsigned)((long long)BH * nkb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dk, (u16 *)dv, BH, N, nblk, c2, scale, dr, vl,
                       wa);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DT, D, false, false, false, true>),
                       dim3((unsigned)((long long)BH * nqb)), dim3(kThreads), 0, stream,
                       (const u16 *)q, (const u16 *)k, (const u16 *)v, (const u16 *)dO,
                       (const float *)ws, (u16 *)dq, BH, N, nblk, nqb, c2, scale, dr, vl, wa);
    return hipGetLastError();
}

typedef hipError_t (*launch_fn)(const void *, const void *, const void *, const void *,
                                const void *, const float *, float *, void *, void *, void *,
                                int, int, float, DropArgs, hipStream_t);

template <int DT, bool DROP>
launch_fn pick_drop(int d, int causal)
{
    if (d == 64) return causal ? launch<DT, 64, true, DROP> : launch<DT, 64, false, DROP>;
    return causal ? launch<DT, 128, true, DROP> : launch<DT, 128, false, DROP>;
}

template <int DT>
launch_fn pick(int d, int causal, bool drop)
{
    return drop ? pick_drop<DT, true>(d, causal) : pick_drop<DT, false>(d, causal);
}


}  // namespace

extern "C" size_t fa_bwd_workspace_size(int B, int H, int N)
{
    if (B < 1 || H < 1 || N < 1) return 0;
    return (size_t)B * (size_t)H * (size_t)((N + kWsRows - 1) / kWsRows) * 2 * kWsRows * sizeof(float);
}

namespace {

// Validation and launch shared by fa_bwd and fa_bwd_dropout.
typedef hipError_t (*launch_window_fn)(const void *, const void *, const void *, const void *,
                                       const void *, const float *, float *, void *, void *,
                                       void *, int, int, WindowArgs, float, hipStream_t);

// Validation shared by fa_bwd, fa_bwd_dropout and fa_bwd_window (win: the
// window sides and the device lengths array, or null).
fa_status run_bwd(const void *q, const void *k, const void *v, const void *o, const void *dO,
                  const float *lse, float *ws, void *dq, void *dk, void *dv, int B, int H,
                  int N, int d, int causal, float scale, fa_dtype dtype, const DropArgs *drop,
                  hipStream_t stream, const WindowArgs *win = nullptr)
{
    if (win && (win->wl < -1 || win->wr < -1)) return FA_ERR_INVALID_ARG;
    if (!q || !k || !v || !o || !dO || !lse || !ws || !dq || !dk || !dv)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (N > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)ws) & 15)
        return FA_ERR_MISALIGNED;
    if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;
    if (win && ((uintptr_t)win->lens & 3)) return FA_ERR_MISALIGNED;

    const long long BH = (long long)B * H;
    const long long nkb = (N + kKeysA - 1) / kKeysA;
    const long long nqb = (N + kQB - 1) / kQB;
    const long long nblk = (N + kWsRows - 1) / kWsRows;
    const long long delta_grid = (BH * nblk * kWsRows + 256 / (d / 8) - 1) / (256 / (d / 8));
    if (BH > INT_MAX || BH * nkb > INT_MAX || BH * nqb > INT_MAX || delta_grid > INT_MAX)
        return FA_ERR_INVALID_ARG;
    const size_t tb = (size_t)BH * (size_t)N * (size_t)d * 2;
    const size_t lb = (size_t)BH * (size_t)N * 4;
    const size_t wb = fa_bwd_workspace_size(B, H, N);
    const void *ins[6] = {q, k, v, o, dO, lse};
    const size_t insz[6] = {tb, tb, tb, tb, tb, lb};
    void *outs[4] = {dq, dk, dv, ws};
    const size_t outsz[4] = {tb, tb, tb, wb};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], outsz[a], ins[b], insz[b])) return FA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], outsz[a], outs[b], outsz[b])) return FA_ERR_INVALID_ARG;
        if (win && win->lens && overlaps(outs[a], outsz[a], win->lens, (size_t)B * 4))
            return FA_ERR_INVALID_ARG;
    }

    if (win) {
        // a side of N or more allows every key on that side (kept inside int)
        const WindowArgs wa = {win->lens, H, win->wl > N ? N : win->wl,
                               win->wr > N ? N : win->wr};
        launch_window_fn wf;
        if (dtype == FA_DTYPE_F16)
            wf = d == 64 ? launch_window<FA_DTYPE_F16, 64> : launch_window<FA_DTYPE_F16, 128>;
        else
            wf = d == 64 ? launch_window<FA_DTYPE_BF16, 64> : launch_window<FA_DTYPE_BF16, 128>;
        if (wf(q, k, v, o, dO, lse, ws, dq, dk, dv, (int)BH, N, wa, scale, stream) != hipSuccess)
            return FA_ERR_LAUNCH;
        return FA_OK;
    }
    launch_fn fn = (dtype == FA_DTYPE_F16) ? pick<FA_DTYPE_F16>(d, causal, drop != nullptr)
                                           : pick<FA_DTYPE_BF16>(d, causal, drop != nullptr);
    const DropArgs dr = drop ? *drop : DropArgs{0u, 0u, 0u, 256u, 1.f};
    if (fn(q, k, v, o, dO, lse, ws, dq, dk, dv, (int)BH, N, scale, dr, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

}  // namespace

extern "C" fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o,
                            const void *dO, const float *lse, float *ws, void *dq, void *dk,
                            void *dv, int B, int H, int N, int d, int causal, float scale,
                            fa_dtype dtype, hipStream_t stream)
{
    return run_bwd(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, dtype,
                   nullptr, stream);
}

extern "C" fa_status fa_bwd_dropout(const void *q, const void *k, const void *v, const void *o,
                                    const void *dO, const float *lse, float *ws, void *dq,
                                    void *dk, void *dv, int B, int H, int N, int d, int causal,
                                    float scale, float p_drop, unsigned long long seed,
                                    unsigned offset, fa_dtype dtype, hipStream_t stream)
{
    if (!(p_drop >= 0.f && p_drop < 1.f)) return FA_ERR_INVALID_ARG;
    const unsigned thr = (unsigned)floor((1.0 - (double)p_drop) * 256.0 + 0.5);
    const DropArgs dr = {(unsigned)seed, (unsigned)(seed >> 32), offset, thr,
                         thr ? 256.f / (float)thr : 0.f};
    return run_bwd(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, dtype, &dr,
                   stream);
}

extern "C" fa_status fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                                   const void *dO, const float *lse, float *ws, void *dq,
                                   void *dk, void *dv, int B, int H, int N, int d,
                                   int window_left, int window_right, const int *seqlens,
                                   float scale, fa_dtype dtype, hipStream_t stream)
{
    const WindowArgs win = {seqlens, H, window_left, window_right};
    return run_bwd(q, k, v, o, dO, lse, ws, dq, dk, dv, B, H, N, d, 0, scale, dtype, nullptr,
                   stream, &win);
}

extern "C" size_t fa_bwd_varlen_workspace_size(int B, int H, int total)
{
    if (B < 1 || H < 1 || total < 1) return 0;
    const size_t wsh = (size_t)kWsRows * ((size_t)(total + kWsRows - 1) / kWsRows + (size_t)B);
    return (size_t)H * wsh * 2 * sizeof(float);
}

extern "C" fa_status fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                                   const void *dO, const float *lse, const int *cu_seqlens,
                                   float *ws, void *dq, void *dk, void *dv, int B, int H,
                                   int total, int max_seqlen, int d, int causal, float scale,
                                   fa_dtype dtype, hipStream_t stream)
{
    if (!q || !k || !v || !o || !dO || !lse || !cu_seqlens || !ws || !dq || !dk || !dv)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || total < 1 || max_seqlen < 1 || max_seqlen > total)
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (max_seqlen > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)ws) & 15)
        return FA_ERR_MISALIGNED;
    if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return FA_ERR_MISALIGNED;
    const long long BH = (long long)B * H;
    const long long cap = ((long long)max_seqlen + kKeysA - 1) / kKeysA * kKeysA;
    const long long wsh = (long long)kWsRows * ((total + kWsRows - 1) / kWsRows + (long long)B);
    constexpr int kMaxRpb = 256 / (64 / 8);
    if (BH > INT_MAX || BH * (cap / kKeysA) > INT_MAX || wsh > INT_MAX ||
        (cap + kMaxRpb - 1) / kMaxRpb > INT_MAX)
        return FA_ERR_INVALID_ARG;
    const size_t tb = (size_t)H * (size_t)total * (size_t)d * 2;
    const size_t lb = (size_t)H * (size_t)total * 4, cb = ((size_t)B + 1) * 4;
    const size_t wb = fa_bwd_varlen_workspace_size(B, H, total);
    const void *ins[7] = {q, k, v, o, dO, lse, cu_seqlens};
    const size_t insz[7] = {tb, tb, tb, tb, tb, lb, cb};
    void *outs[4] = {dq, dk, dv, ws};
    const size_t outsz[4] = {tb, tb, tb, wb};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 7; ++b)
            if (overlaps(outs[a], outsz[a], ins[b], insz[b])) return FA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], outsz[a], outs[b], outsz[b])) return FA_ERR_INVALID_ARG;
    }
    const VarlenArgs vl = {cu_seqlens, H, (int)cap, (int)wsh};
    launch_varlen_fn fn = (dtype == FA_DTYPE_F16) ? pick_varlen<FA_DTYPE_F16>(d, causal)
                                                  : pick_varlen<FA_DTYPE_BF16>(d, causal);
    if (fn(q, k, v, o, dO, lse, ws, dq, dk, dv, (int)BH, total, vl, scale, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}
