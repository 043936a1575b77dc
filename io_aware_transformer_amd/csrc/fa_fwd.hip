// fa_fwd.hip -- exact attention forward pass for MI355X (gfx950, CDNA4).
//
// Pages cited (by tag and section):
//   [P-notes] "FlashAttention v1 & v2 笔记"            (yiran529.github.io)
//   [P-baidu] "FlashAttention 优化原理与实现要点解析"    (cloud.baidu.com)
//   [P-wmrh]  "FlashAttention V2 核心原理与架构设计"     (wmrh.cn)
//
// Work decomposition.  The grid runs over (batch, head, Q block)
// ([P-notes] §五.1: parallelism along the sequence as well).  A work-group
// owns 256 query rows and walks the keys with the Q block outer and the K/V
// block inner ([P-notes] §五.2, [P-wmrh] §2.2 "V2"), so its output is
// accumulated on chip and written once.  Each of its eight wavefronts owns a
// 32-row slab of the queries ([P-notes] §五.3, split-Q): softmax statistics
// never leave the wave and no cross-wave reduction exists.  K/V move through
// LDS in tiles of 128 keys, double buffered, and each tile is consumed as
// two compute steps of 64 keys.
//
// Per 64-key step j, per wave ([P-baidu] §5 steps 1-4, §4.2, §4.3):
//   S^T = K_j Q^T                 MFMA 32x32x16, 16-bit in, fp32 accumulate
//   mask                          diagonal and ragged-tail steps only
//   m' = max(m, rowmax(S) c)      c = |scale| log2(e); log2 domain
//   P = 2^(S c - m'),  l = 2^(m - m') l + rowsum(P)
//   O^T = 2^(m - m') O^T + V_j^T P^T      MFMA, P rounded to 16 bits
// and after the last step O = O / l, lse = (m + log2 l) ln 2 ([P-baidu] §4.3
// and §6: numerator and denominator kept apart, one division at the end).
//
// MI355X-specific choices (the pages' A100 design is prior art only):
//  * S^T rather than S.  In the 32x32 MFMA output a lane holds 16 keys of ONE
//    query column (lane l and l+32 share the column).  Row max and row sum are
//    per-lane work plus one v_permlane32_swap, and the fp32 scores, once
//    rounded to 16 bits, are already the B operand of the P.V product.
//  * Every accumulator lives in VGPRs (about 178 per lane), so two waves
//    share each SIMD and one issues while the other waits on LDS or on the
//    matrix pipe.  (Measured: plain VALU work of one wave overlaps the other
//    wave's MFMAs, about 30% slower than alone, but v_dot2 instructions wait
//    for the matrix pipe, and VALU work between one wave's own MFMAs adds to
//    their time.  A schedule that alternates the two waves' MFMA and softmax
//    phases kept the pipe busier but ran the power-limited chip at a lower
//    clock and was not faster at the same accuracy.)  One 8-wave work-group
//    fills a CU (128 KB of LDS); the 128-key tiles halve the barriers per key
//    against 64-key tiles.
//    Measured on MI355X and rejected: 4-wave work-groups (two per CU), a
//    12-wave group at three waves per SIMD, an in-wave software pipeline
//    (S(j+1) on MFMA under softmax(j)), and a V^T copy of each tile in LDS
//    for b128 operand reads (its extra barrier cost more than it saved).
//  * MFMA operand reads from LDS are issued a fixed number of MFMAs ahead
//    and the interleave is pinned with scheduling-group barriers; left
//    alone, the scheduler moves each read next to its MFMA and the wave
//    stalls on LDS latency.
//  * K/V tiles go HBM -> LDS with buffer_load ... lds (no registers, no VALU);
//    rows past N come back as zeros from the buffer range check.  Each wave's
//    share of the next tile's loads is spread over the MFMAs of the tile's
//    first QK^T rather than queued all at once, which stalled every wave on
//    the vector-memory path at the start of each tile.  K is read with
//    ds_read_b128, V with ds_read_b64_tr_b16, which delivers V^T fragments
//    directly.  16-byte chunks inside each row are XOR-swizzled so both read
//    patterns are bank-conflict free.
//  * The reference maximum m moves only when a step's maximum exceeds it by
//    more than 8 (log2 units); then P <= 256 and the result is the same
//    quotient, while the O rescale (64 multiplies per lane) is almost never
//    executed.  For binary16 the reference sits a further 7 below (see
//    kF16Lift), so tiny weights do not round to zero.  Row reductions run as
//    trees (v_max3) or several independent chains, never one serial
//    dependency chain.
//  * O leaves through LDS: each wave stages its 32 rows in the idle K
//    buffers and stores whole 16-byte row chunks, 4 (d128) or 8 (d64)
//    complete rows per instruction.
//
// Causal K/V tiles wholly above the diagonal are never visited ([P-baidu]
// §7); the last Q block of a ragged N masks keys >= N and stores no rows >= N.
//
// One kernel template serves every forward entry point: MODE 0 / 1 (all
// keys / causal: fa_fwd), 2 (sliding window and valid lengths, the mask
// kinds of [P-baidu] §8: fa_fwd_window), 3 (one key segment per grid row,
// merged by fa_fwd_merge_kernel: fa_fwd_split, fa_fwd_split_noalloc, and
// fa_fwd_decode, whose key sequence may be longer than the rows), 4 / 5 (all keys / causal
// over packed variable-length sequences, the padding kind of [P-baidu] §8
// without the padding: fa_fwd_varlen), and the DROP flag on modes 0 / 1
// (dropout fused into the kernel, [P-wmrh] §1.2: fa_fwd_dropout).
// Each variant is a compile-time instantiation, so the tuned full and causal
// kernels carry none of the others' code.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>
#include <mutex>

#include "fa_fwd.h"

namespace {

typedef unsigned short u16;
typedef u16 u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;                 // one 32-column MFMA block
constexpr int kBR = kWaves * kRowsPerWave;       // query rows per work-group
constexpr int kBC = 64;                          // keys per compute step
constexpr int kLT = 128;                         // keys per LDS tile
constexpr int kNSub = kLT / kBC;                 // compute steps per LDS tile
constexpr float kLazy = 8.0f;                    // reference-max slack, log2 units
// For binary16 the reference is kept kF16Lift (log2 units) below the running
// row maximum: the weights are lifted by 2^kF16Lift, the largest then being
// 2^(kLazy + kF16Lift) = 2^15 < 65504, and a weight 2^-31 below the row
// maximum still rounds to a nonzero binary16.  Against the maximum itself,
// everything under 2^-25 would round to 0: a flat tail of 2^20 keys each 18
// nats under a dominant key (about 1.6% of the row) would vanish.  The lift
// cancels in O (numerator and row sums carry it alike) and in lse (which is
// the reference plus the log of the lifted sum).
constexpr float kF16Lift = 7.0f;
constexpr int kQkAhead = 4;                      // K operand reads in flight (MFMAs)
constexpr int kPvAhead = 3;                      // V operand reads in flight (MFMAs)
constexpr unsigned kRsrcWord3 = 0x00020000u;     // raw buffer, 32-bit data

// Element-type specifics: the MFMA and fp32 -> 16-bit pair conversion
// (round to nearest even).
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
    // acc + the two 16-bit values of a packed pair (products by 1.0 are exact)
    static __device__ __forceinline__ float sum2(unsigned pr, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), one, acc, false);
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
    static __device__ __forceinline__ float sum2(unsigned pr, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), one, acc, false);
    }
};

// Geometry of one K or V tile (kLT rows of D 16-bit elements) in LDS: rows
// are dense, 16-byte chunks inside a row are XOR-swizzled by a function of
// the row.  K rows: 16 consecutive rows reading one logical chunk (one
// ds_read_b128 per lane) land on distinct banks.  V rows: the 4 rows x 64
// bytes that 32 lanes of one transposing read touch land on distinct banks.
template <int D> struct Tile {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kChunks = D / 8;
    static constexpr int kBytes = kLT * kRowBytes;
    static constexpr int kLoads = kBytes / 1024;                       // 1 KB loads per tile
    static constexpr int kLoadsPerWave = kLoads / kWaves;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static __device__ __forceinline__ int kswz(int row) {
        return D == 128 ? (row & 15) : ((row >> 1) & 7);
    }
    static __device__ __forceinline__ int vswz(int row) {
        return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    }
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Compile-time buffer index (the K/V LDS buffers are separate objects and
// always selected statically, so the compiler can tell that the HBM->LDS
// prefetch of one buffer does not alias the reads of another and need not
// wait for it).
template <int I> struct Buf { static constexpr int value = I; };
template <bool B> struct Flag { static constexpr bool value = B; };

// v_max3_f32 / v_max_f32 without the input canonicalisation the compiler
// adds to fmaxf in IEEE mode (scores are never signalling NaNs).
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Maximum of N values as a tree of three-input maxima (depth log3 N): each
// level takes the values three at a time and carries the one or two left
// over to the next level, so N values cost ceil((N - 1) / 2) instructions.
template <int N> struct TreeMax {
    static __device__ __forceinline__ float of(const float (&a)[N]) {
        constexpr int T = N / 3, M = T + N % 3;
        float b[M];
#pragma unroll
        for (int i = 0; i < T; ++i) b[i] = max3(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
#pragma unroll
        for (int i = T; i < M; ++i) b[i] = a[3 * T + (i - T)];
        return TreeMax<M>::of(b);
    }
};
template <> struct TreeMax<2> {
    static __device__ __forceinline__ float of(const float (&a)[2]) { return max2(a[0], a[1]); }
};
template <> struct TreeMax<1> {
    static __device__ __forceinline__ float of(const float (&a)[1]) { return a[0]; }
};

// Key (row) position held by accumulator register r of a 32x32 MFMA output
// in wave half hh: 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Value of x in the other half of the wave (lane l <-> l^32), via
// v_permlane32_swap: swap(x, x) yields [x_lo, x_lo] and [x_hi, x_hi].
__device__ __forceinline__ float half_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products
// with the multipliers 0xD2511F53 (word 0) and 0xCD9E8D57 (word 2), the high
// halves XORed with the other words and the key, the key bumped by the Weyl
// constants (0x9E3779B9, 0xBB67AE85) between rounds.  The key is uniform
// over the grid, so its schedule stays in scalar registers.
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

// Dropout parameters of one launch: a weight is kept when its random byte is
// below thr, and the kept weights are scaled by fscale = 256 / thr.
struct DropArgs {
    unsigned seed_lo, seed_hi, offset, thr;
    float fscale;
};

// MODE 0: every key; 1: causal (key <= query); 2: window and valid lengths,
// key j allowed for query i of batch element b when
// max(0, i - wl) <= j <= min(L_b - 1, i + wr) (wl / wr < 0: that side open;
// L_b = LENS[b] clamped to [0, N], or N without LENS); rows i >= L_b have no
// keys and get o = 0, lse = -inf.  3: one key segment [kseg*y, kseg*(y+1))
// (y = blockIdx.y) of the window rule with L_b = N; writes the segment's
// normalised O in fp32 to PO and its lse to PL ([y][b*H+h][row]), rows
// without keys in the segment 0 and -inf, for a merge kernel to combine.
// With wsplit = 2 and N <= 32 rows, waves 0 and 1 each take every other
// 64-key step of the segment's tiles and write it as segment 2y + w.
// Modes 0 and 1 ignore H, wl, wr, LENS, kseg, wsplit, PO, PL.  4 / 5: modes 0 / 1
// over packed variable-length sequences: N is the token count of each head
// ([H, N, d] tensors), LENS the cumulative sequence starts (B + 1 values),
// BH = B*H, and work-group (b*H + h, Q block) works on sequence b of head h,
// rows [LENS[b], LENS[b+1]) of the head (bounds clamped to [0, N] and the
// length to nqb Q blocks, so no access leaves the tensors).
//
// DROP (modes 0 and 1 only): dropout on the normalised weights.  Weight
// (b*H+h, i, j) is kept when byte 4*((j%32)/8) + j%4 of Philox4x32-10 with
// counter (i, 2*(j/32) + (j/4)%2, b*H+h, offset) and key (seed low word,
// seed high word) is below dr.thr; kept weights are scaled by dr.fscale.
// The row sum and lse are those of the undropped weights.  In the MFMA
// layout a lane's 16 keys of one 32-key block are exactly the 16 bytes of
// one call (key 8g + 4hh + e is byte 4g + e), so a lane makes one call per
// 32 keys and no random number is shared between lanes.
template <int DT, int D, int MODE, bool DROP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const u16 *__restrict__ Q, const u16 *__restrict__ K,
                   const u16 *__restrict__ V, u16 *__restrict__ O,
                   float *__restrict__ LSE, int BH, int N_in, int nqb, float c,
                   unsigned qand, unsigned qxor, int H, int wl, int wr,
                   const int *__restrict__ LENS, int kseg, int nk_in, int wsplit,
                   float *__restrict__ PO, float *__restrict__ PL, DropArgs dr)
{
    static_assert(!DROP || MODE <= 1, "dropout is built for the full and causal masks");
    constexpr bool VARLEN = MODE >= 4;
    constexpr bool CAUSAL = MODE == 1 || MODE == 5;
    constexpr bool GEN = MODE == 2 || MODE == 3;
    constexpr bool SPLIT = MODE == 3;
    // the fp32 row sum is kept for bfloat16 and under dropout (where the
    // weights applied to V no longer sum to the normaliser)
    constexpr bool FSUM = DT == FA_DTYPE_BF16 || DROP;
    using E = Elem<DT>;
    using T = Tile<D>;
    constexpr int KT = D / 16;    // MFMA k-steps over d
    constexpr int DB = D / 32;    // 32-row blocks of O^T
    constexpr int PT = kBC / 16;  // MFMA k-steps over the keys of a tile
    constexpr int NKB = kBC / 32; // 32-key blocks of S^T per tile

    __shared__ __attribute__((aligned(1024))) unsigned char k0s[T::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char k1s[T::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char v0s[T::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char v1s[T::kBytes];
    // buffers: 0,1 = K tiles (j even/odd), 2,3 = V tiles (j even/odd)
    auto bufp = [&](auto b) -> LDS unsigned char * {
        constexpr int i = decltype(b)::value;
        if constexpr (i == 0) return (LDS unsigned char *)k0s;
        else if constexpr (i == 1) return (LDS unsigned char *)k1s;
        else if constexpr (i == 2) return (LDS unsigned char *)v0s;
        else return (LDS unsigned char *)v1s;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
#ifdef FA_DEBUG_LDS_POISON
    // Race-check build: every LDS byte starts as an all-ones (NaN) pattern,
    // so an operand read that overtook its tile load, or a tile read after
    // its buffer was refilled, turns the outputs into NaN or changes them.
    {
        const u32x4 nan4 = {~0u, ~0u, ~0u, ~0u};
        for (int i = tid; i < T::kBytes / 16; i += kThreads) {
            ((LDS u32x4 *)k0s)[i] = nan4;
            ((LDS u32x4 *)k1s)[i] = nan4;
            ((LDS u32x4 *)v0s)[i] = nan4;
            ((LDS u32x4 *)v1s)[i] = nan4;
        }
        __syncthreads();
    }
#endif
#ifdef FA_DEBUG_SERIAL_TILES
    // Race-check build: tile t+1 is loaded only after tile t is done
    // (loads, wait, barrier), so no load overlaps any read
    constexpr bool kSerial = true;
#else
    constexpr bool kSerial = false;
#endif
    // wave index (kRowsPerWave query rows each).  At d = 128 it is held in a
    // scalar register, so tile-load addressing stays on the scalar unit (at
    // d = 64 that measured no faster)
    const int w = D == 128 ? __builtin_amdgcn_readfirstlane(tid >> 6) : (tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // Work-group -> (batch*head, Q block).  Heads vary fastest: with
    // work-groups dealt round-robin over the 8 XCDs, all Q blocks of one head
    // share an XCD (and its L2) whenever B*H is a multiple of 8.  Causal
    // grids start with the longest (last) Q blocks.
    const int L = blockIdx.x;
    const int bh = L % BH;
    const int qblk = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
    // N: rows of this work-group's attention problem; row0: its first row in
    // the [rows, d] view of the tensors
    int N = N_in;
    size_t row0 = (size_t)bh * (size_t)N_in;
    if constexpr (VARLEN) {
        const int b = bh / H, h = bh % H;
        const int start = min(max(LENS[b], 0), N_in);
        const int end = min(max(LENS[b + 1], start), N_in);
        N = min(end - start, nqb * kBR);
        row0 = (size_t)h * (size_t)N_in + (size_t)start;
        if (qblk * kBR >= N) return;                   // Q block past the sequence
    }
    const size_t head = row0 * D;
    // keys of the problem: mode 3 may run the rows against a separate key
    // sequence of nk_in rows per head (decoding shapes); elsewhere the keys
    // are the rows themselves
    const int NKEYS = SPLIT ? nk_in : N;
    const size_t khead = SPLIT ? (size_t)bh * (size_t)NKEYS * D : head;
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void *)(Q + head), 0, N * T::kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(K + khead), 0, NKEYS * T::kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(V + khead), 0, NKEYS * T::kRowBytes, kRsrcWord3);

    // Mode 3 with wsplit = 2 and at most kRowsPerWave rows (decoding shapes,
    // where only the first wave would have rows): waves 0 and 1 both take
    // those rows and compute alternate kBC-key steps of every LDS tile, each
    // as a key segment of its own (partials slot 2y + w for y = blockIdx.y),
    // so two SIMDs share the tile's compute; the other waves only load.
    const bool dsplit = SPLIT && wsplit > 1 && N <= kRowsPerWave;
    const bool writer = !dsplit || w < 2;           // this wave stores results
    const int seg = dsplit ? 2 * (int)blockIdx.y + (w & 1) : (int)blockIdx.y;
    const int q0 = qblk * kBR + kRowsPerWave * (dsplit ? 0 : w);   // first row of the wave
    const int qrow = q0 + l32;                      // the query row of this lane

    // Q slab -> B-operand fragments (rows past N read as zero), kept in
    // registers for the whole loop.  qand/qxor zero or negate Q exactly.
    u16x8 qf[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        const int off = (qrow * D + 16 * kk + 8 * hh) * 2;
        u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        x = (x & qand) ^ qxor;
        qf[kk] = __builtin_bit_cast(u16x8, x);
    }

    const int n_keys_tiles = (N + kBC - 1) / kBC;      // compute steps over all keys
    const int n_steps = CAUSAL ? min(n_keys_tiles, (qblk + 1) * (kBR / kBC)) : n_keys_tiles;
    int t_begin = 0;                                   // LDS tiles [t_begin, n_tiles)
    int n_tiles = (n_steps + kNSub - 1) / kNSub;       // of kLT keys
    // steps this wave computes: causal rows q0..q0+31 need keys <= q0+31
    const int n_w = (q0 >= N) ? 0 : (CAUSAL ? min(n_steps, (q0 + kRowsPerWave - 1) / kBC + 1)
                                            : n_steps);
    // MODE 2: valid length of this batch element, the work-group's and this
    // wave's key ranges (in steps j_lo..j_hi), and the per-lane key bounds
    // len: valid rows (and keys, except in mode 3, where klen = NKEYS)
    int len = N, klen = N, j_lo = 0, j_hi = -1, klo_row = 0, khi_row = -1, kbeg = 0, kend = N;
    // rows without keys: o = 0 / lse = -inf (or the fp32 partials in mode 3)
    const size_t prow = ((size_t)seg * BH + bh) * N + qrow;
    auto write_empty = [&]() {
        if (!writer) return;
        if constexpr (SPLIT) {
            float *po = PO + prow * D;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) *(f32x4 *)(po + 32 * db + 8 * g + 4 * hh) = z;
            if (hh == 0) PL[prow] = neg_inf();
        } else {
            u16 *orow = O + head + (size_t)qrow * D;
            const u32x2 z = {0u, 0u};
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) *(u32x2 *)(orow + 32 * db + 8 * g + 4 * hh) = z;
            if (hh == 0) LSE[row0 + qrow] = neg_inf();
        }
    };
    if constexpr (GEN) {
        len = LENS ? min(max(LENS[bh / H], 0), N) : N;
        klen = SPLIT ? NKEYS : len;
        if constexpr (SPLIT) {
            kbeg = blockIdx.y * kseg;
            kend = min(klen, kbeg + kseg);
        }
        const int r0 = qblk * kBR, r1 = min(r0 + kBR, len) - 1;
        const int klo = max(wl < 0 ? 0 : max(0, r0 - wl), kbeg);
        const int khi = min(wr < 0 ? klen - 1 : min(klen - 1, r1 + wr), kend - 1);
        if (r0 > r1 || klo > khi) {                    // no (row, key) pair in the work-group
            // (mode 3: no row of this work-group reaches the segment, and the
            // merge reads a row's segments only up to its last allowed key)
            if (!SPLIT && qrow < N) write_empty();
            return;
        }
        t_begin = (klo / kBC) / kNSub;
        n_tiles = (khi / kBC) / kNSub + 1;
        if (q0 < len) {
            const int w1 = min(q0 + kRowsPerWave, len) - 1;
            const int wlo = max(wl < 0 ? 0 : max(0, q0 - wl), kbeg);
            const int whi = min(wr < 0 ? klen - 1 : min(klen - 1, w1 + wr), kend - 1);
            if (wlo <= whi) {
                j_lo = wlo / kBC;
                j_hi = whi / kBC;
            }
        }
        klo_row = max(wl < 0 ? 0 : qrow - wl, kbeg);
        khi_row = min(wr < 0 ? klen - 1 : min(klen - 1, qrow + wr), kend - 1);
    }

    // ---- HBM -> LDS tile loads (each wave moves its share, 1 KB per load)
    // One of this wave's 1 KB loads of a tile: n < kLoadsPerWave is K, the
    // rest V.  base = byte offset of the tile's first row; a base at or past
    // 2^30 (>= every head's size) makes every lane out of range, which fills
    // the LDS destination with zeros without touching memory.
    static_assert(T::kLoads % kWaves == 0, "whole loads per wave");
    // Load li covers rows li*kRowsPerLoad.., and kWaves*kRowsPerLoad is a
    // multiple of 16, so a lane's swizzled byte offset inside its 1 KB does
    // not depend on jn: it is computed once (kl / vl) and each load adds the
    // wave-uniform part base + li*1024.
    static_assert((kWaves * T::kRowsPerLoad) % 16 == 0, "swizzle invariant over loads");
    const int lrow = w * T::kRowsPerLoad + lane / T::kChunks;   // row of load jn = 0
    const int kl = (lane / T::kChunks) * T::kRowBytes + (((lane % T::kChunks) ^ T::kswz(lrow)) << 4);
    const int vl = (lane / T::kChunks) * T::kRowBytes + (((lane % T::kChunks) ^ T::vswz(lrow)) << 4);
    auto issue_one = [&](int n, auto kbuf, auto vbuf, int base) {
        const bool is_v = n >= T::kLoadsPerWave;
        const int jn = is_v ? n - T::kLoadsPerWave : n;
        const int li = jn * kWaves + w;
        const int off = (base + li * 1024) + (is_v ? vl : kl);
        if (is_v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (LDS void *)(bufp(vbuf) + li * 1024), 16, off, 0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (LDS void *)(bufp(kbuf) + li * 1024), 16, off, 0, 0, 0);
    };

    // Per-lane LDS offsets of the MFMA operand reads (loop invariant).
    int koff[KT];           // K_j: row 32*kb + l32, logical chunk 2*kk + hh
#pragma unroll
    for (int kk = 0; kk < KT; ++kk)
        koff[kk] = l32 * T::kRowBytes + (((2 * kk + hh) ^ T::kswz(l32)) << 4);
    int voff[DB];           // V_j transposing reads, see the layout note above
    {
        const int g = lane >> 4, i = lane & 15;
        const int row = 4 * (g >> 1) + (i >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 32 * db + 16 * (g & 1) + 4 * (i & 3);
            voff[db] = row * T::kRowBytes + (((d >> 3) ^ T::vswz(row)) << 4) + ((d >> 2) & 1) * 8;
        }
    }

    // Per-lane V read addresses of each V buffer, formed once and held in
    // registers (the empty asm keeps the compiler from re-forming them): every
    // transposing read is then one of them plus an immediate offset.  Formed
    // per read, each cost a VALU op, as the V buffers lie beyond the 64 KB
    // reach of the offset field.  The price: the compiler no longer knows
    // which buffer such a read touches, so it waits for this wave's in-flight
    // tile loads before the first V read of a step; those loads were issued a
    // whole QK^T earlier and have landed, and the trade measured faster.
    // (At d = 64 the tiles are half as large and holding them measured slower.)
    const LDS unsigned char *vad[2][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        vad[0][db] = bufp(Buf<2>{}) + voff[db];
        vad[1][db] = bufp(Buf<3>{}) + voff[db];
        if constexpr (D == 128) asm volatile("" : "+v"(vad[0][db]), "+v"(vad[1][db]));
    }

    int sub = 0;   // which kBC-key half of the LDS tile the current step uses
    auto kfrag = [&](auto buf, int kb, int kk) -> u16x8 {
        return *(const LDS u16x8 *)(bufp(buf) + (sub * kBC + kb * 32) * T::kRowBytes + koff[kk]);
    };
    auto vfrag = [&](auto buf, int db, int kk) -> u16x8 {
        constexpr int vb = decltype(buf)::value - 2;
        const LDS unsigned char *p = vad[vb][db] + (sub * kBC + kk * 16) * T::kRowBytes;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS s16x4 *)(p + 8 * T::kRowBytes));
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // S^T(j) = K_j Q^T: s[kb], keys 32*kb.., query column l32.  Operand
    // i (k-step i / NKB, key block i % NKB) is read from LDS kQkAhead MFMAs
    // before its MFMA; the schedule is pinned (one read per MFMA) so the
    // compiler cannot pull the reads up against their uses.  With loads, this
    // wave's share of the next tile's HBM -> LDS loads rides along, one load
    // every NR / NLD MFMAs, instead of all waves queueing them at once.
    auto qk = [&](f32x16 (&s)[NKB], auto buf, auto loads, auto kbuf, auto vbuf, int base) {
        constexpr bool LD = decltype(loads)::value;
        constexpr int NR = KT * NKB;
        constexpr int AH = kQkAhead;
        constexpr int NLD = 2 * T::kLoadsPerWave;
        static_assert(NR % NLD == 0, "loads spread evenly over the MFMAs");
        constexpr int ST = NR / NLD;
        u16x8 kf[NR];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < AH; ++i) kf[i] = kfrag(buf, i % NKB, i / NKB);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (i + AH < NR) kf[i + AH] = kfrag(buf, (i + AH) % NKB, (i + AH) / NKB);
            const int kb = i % NKB, kk = i / NKB;
            if (kk == 0) {
                const f32x16 z = {};
                s[kb] = E::mfma(kf[i], qf[kk], z);
            } else {
                s[kb] = E::mfma(kf[i], qf[kk], s[kb]);
            }
            if (LD && i % ST == 0) issue_one(i / ST, kbuf, vbuf, base);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);      // DS reads
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            if (i < NR - AH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (LD && i % ST == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    auto mask = [&](f32x16 (&s)[NKB], int t) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t * kBC + 32 * kb + acc_row(r, hh);
                bool keep;
                if constexpr (GEN) keep = key >= klo_row && key <= khi_row;
                else keep = key < N && (!CAUSAL || key <= qrow);
                if (!keep) s[kb][r] = neg_inf();
            }
    };

    float m = neg_inf();   // reference max, log2 domain (kF16Lift below the maximum for binary16)
    float l = 0.f;         // this lane's half of the row sum of P (fp32)
    float lh = 0.f;        // the same sum of P rounded to 16 bits
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

    // Row max of S(j) and the (lazy) update of the reference max.
    auto update_max = [&](f32x16 (&s)[NKB]) {
        float v[NKB * 16];
#pragma unroll
        for (int i = 0; i < NKB * 16; ++i) v[i] = s[i >> 4][i & 15];
        const float mx = TreeMax<NKB * 16>::of(v);
        const float mt = half_max(mx) * c;
        constexpr float lift = (DT == FA_DTYPE_F16) ? kF16Lift : 0.f;
        if (__builtin_amdgcn_ballot_w64(mt > m + (kLazy + lift))) {
            const float mn = fmaxf(m, mt - lift);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m - mu);
            if constexpr (FSUM) l *= alpha;
            if constexpr (!DROP) lh *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m = mn;
        }
    };

    // P(j) = 2^(S c - m) rounded to 16 bits (B operand of P.V), row sums.
    // O is divided by the sum of the ROUNDED weights, so the weights applied
    // to V stay a convex combination (the rounding of a dominant weight
    // cancels).  lse uses the fp32 sum for bfloat16; for binary16 the
    // rounded sum is within 2^-11 relative of it (|lse error| <= 4.9e-4),
    // so it serves for both.
    auto softmax = [&](f32x16 (&s)[NKB], u32x4 (&pk)[PT], int j) {
        const float mu = (m == neg_inf()) ? 0.f : m;
        float rs[4], rh[4];
        // dropout bytes: one Philox call per 32-key block (see DROP above)
        u32x4 rnd[NKB];
        if constexpr (DROP) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                rnd[kb] = philox4x32_10((unsigned)qrow, (unsigned)(2 * (j * NKB + kb) + hh),
                                        (unsigned)bh, dr.offset, dr.seed_lo, dr.seed_hi);
        }
        // groups of 8 scores: 8 FMAs, 8 exps, then sums and packing, so the
        // temporaries die inside the group (scheduling barrier per group)
#pragma unroll
        for (int g = 0; g < 2 * NKB; ++g) {
            const int kb = g >> 1, r0 = (g & 1) * 8;
            float x[8], p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = fmaf(s[kb][r0 + e], c, -mu);
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(x[e]);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (FSUM) {
                    const float a = p[2 * h] + p[2 * h + 1];
                    rs[h] = (g == 0) ? a : rs[h] + a;
                }
                if constexpr (DROP) {
                    // register r holds key 8(r/4) + 4hh + r%4: byte r of the
                    // call.  The pair's two bytes (r = r0 + 2h, r0 + 2h + 1)
                    // are spread into the two 16-bit halves of a word; byte -
                    // thr is negative exactly for a kept weight, so the
                    // arithmetic shift by 15 turns each half into an all-ones
                    // (kept) or all-zeros (dropped) mask of its packed weight.
                    // (v_perm_b32(a, b, sel): selector byte 0-3 takes byte
                    // 0-3 of b, 0x0c a zero byte)
                    const unsigned wd = rnd[kb][(r0 >> 2) + (h >> 1)];
                    const unsigned two = __builtin_amdgcn_perm(0u, wd, (h & 1) ? 0x0c030c02u : 0x0c010c00u);
                    s16x2 keep = __builtin_bit_cast(s16x2, two) - (short)dr.thr;
                    keep = keep >> 15;
                    pk[2 * kb + (r0 >> 3)][h] =
                        E::pack2(p[2 * h], p[2 * h + 1]) & __builtin_bit_cast(unsigned, keep);
                } else {
                    const unsigned pr = E::pack2(p[2 * h], p[2 * h + 1]);
                    rh[h] = E::sum2(pr, (g == 0) ? 0.f : rh[h]);
                    pk[2 * kb + (r0 >> 3)][h] = pr;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FSUM) l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        if constexpr (!DROP) lh += (rh[0] + rh[1]) + (rh[2] + rh[3]);
    };

    // O^T += V_j^T P(j)^T, operand i (k-step i / DB, d block i % DB) read
    // kPvAhead MFMAs ahead, schedule pinned as in qk (two reads per MFMA)
    auto pv = [&](auto buf, u32x4 (&pk)[PT]) {
        constexpr int NM = PT * DB;
        constexpr int AH = kPvAhead;
        u16x8 vf[NM];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < AH; ++i) vf[i] = vfrag(buf, i % DB, i / DB);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i + AH < NM) vf[i + AH] = vfrag(buf, (i + AH) % DB, (i + AH) / DB);
            oacc[i % DB] = E::mfma(vf[i], __builtin_bit_cast(u16x8, pk[i / DB]), oacc[i % DB]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < NM - AH; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    auto tile_masked = [&](int t) {
        bool mk;
        if constexpr (GEN) {
            // every row of the wave keeps every key of the step?
            const int w1 = q0 + kRowsPerWave - 1;
            const bool lo_ok = t * kBC >= max(wl < 0 ? 0 : w1 - wl, kbeg);
            const bool hi_ok = t * kBC + kBC - 1 <=
                               min(wr < 0 ? klen - 1 : min(klen - 1, q0 + wr), kend - 1);
            mk = !(lo_ok && hi_ok);
        } else {
            mk = (CAUSAL && t * kBC + kBC - 1 > q0) || (t * kBC + kBC > N);
        }
        // At d = 128 the wave index, and with it every operand of mk, is
        // already scalar, so the flag stays on the scalar unit; at d = 64 it
        // is made uniform explicitly.
        if constexpr (D == 128) return mk;
        return __builtin_amdgcn_readfirstlane((int)mk) != 0;
    };

    // ---- tile loop.  LDS tile t (kLT keys: K_t in k[t%2], V_t in v[t%2]) is
    // computed as kNSub steps of kBC keys, j = kNSub*t + u, each
    // QK^T(j) -> max -> softmax -> P(j).V.  Tile t+1 streams into the other
    // buffers during step u = 0 (those were last read in tile t-1, before the
    // barrier that ended it); waves that skip the step still issue their
    // share.  After the last tile the loads are aimed out of range (zero
    // fill of a buffer nobody reads, no memory traffic).
#pragma unroll
    for (int n = 0; n < 2 * T::kLoadsPerWave; ++n)
        issue_one(n, Buf<0>{}, Buf<2>{}, t_begin * kLT * T::kRowBytes);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 sc[NKB];
    auto tile = [&](auto par, int t) {
        constexpr int P = decltype(par)::value;
        const int base = (t + 1 < n_tiles) ? (t + 1) * kLT * T::kRowBytes : (1 << 30);
#pragma unroll
        for (int u = 0; u < kNSub; ++u) {
            const int j = kNSub * t + u;
            bool run;
            if constexpr (GEN) run = j >= j_lo && j <= j_hi && (!dsplit || u == w);
            else run = j < n_w;
            if (run) {
                sub = u;
                u32x4 pk[PT];
                __builtin_amdgcn_s_setprio(2);
                if (u == 0) qk(sc, Buf<P>{}, Flag<!kSerial>{}, Buf<1 - P>{}, Buf<3 - P>{}, base);
                else qk(sc, Buf<P>{}, Flag<false>{}, Buf<1 - P>{}, Buf<3 - P>{}, base);
                __builtin_amdgcn_s_setprio(0);
                if (tile_masked(j)) mask(sc, j);
                update_max(sc);
                softmax(sc, pk, j);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(2);
                pv(Buf<2 + P>{}, pk);
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
            } else if (u == 0 && !kSerial) {
#pragma unroll
                for (int n = 0; n < 2 * T::kLoadsPerWave; ++n)
                    issue_one(n, Buf<1 - P>{}, Buf<3 - P>{}, base);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (kSerial) {
#pragma unroll
            for (int n = 0; n < 2 * T::kLoadsPerWave; ++n)
                issue_one(n, Buf<1 - P>{}, Buf<3 - P>{}, base);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    };

    for (int t = t_begin; t < n_tiles; t += 2) {
        tile(Buf<0>{}, t);
        if (t + 1 < n_tiles) tile(Buf<1>{}, t + 1);
    }

    // ---- epilogue: one division per row, 16-bit O, fp32 lse
    if constexpr (GEN) {
        if (qrow >= len && qrow < N) write_empty();    // rows without keys
    }
    if constexpr (SPLIT) {
        // the segment's normalised O in fp32 and its lse; rows that met no
        // key of the segment (row sum 0) are empty
        if (writer && q0 < len) {
            const float lht = half_sum(lh);
            const float lt = (DT == FA_DTYPE_BF16) ? half_sum(l) : lht;
            if (qrow < len) {
                if (lht > 0.f) {
                    const float inv = 1.f / lht;
                    float *po = PO + prow * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            f32x4 x;
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * g + e] * inv;
                            *(f32x4 *)(po + 32 * db + 8 * g + 4 * hh) = x;
                        }
                    if (hh == 0) PL[prow] = (m + log2f(lt)) * 0.69314718055994530942f;
                } else {
                    write_empty();
                }
            }
        }
        return;
    }
    if (GEN ? (q0 < len) : (n_w > 0)) {
        // under dropout O is the kept weights' sum scaled by fscale over the
        // undropped fp32 row sum; otherwise over the rounded-weight sum
        const float lht = DROP ? 0.f : half_sum(lh);
        const float lt = FSUM ? half_sum(l) : lht;
        const float inv = DROP ? dr.fscale / lt : 1.f / lht;
        // O leaves through this wave's own 32-row slice of the idle K
        // buffers (the loop's last barrier has retired every tile read and
        // load): a lane holds 4 consecutive columns of its row per (db, g),
        // i.e. half of 16-byte chunk 4*db + g of that row.  Read back as whole
        // chunks, one store instruction writes 64 * 16 / (2 * D) complete
        // consecutive rows, a contiguous run of the head's row-major O.
        // Chunks are XOR-swizzled by row so each LDS access spreads over the
        // banks.
        constexpr int CH = T::kChunks;                    // 16-byte chunks per row
        LDS unsigned char *stage = (w < kWaves / 2 ? bufp(Buf<0>{}) : bufp(Buf<1>{})) +
                                   (w % (kWaves / 2)) * (kRowsPerWave * T::kRowBytes);
        static_assert((kWaves / 2) * kRowsPerWave * T::kRowBytes <= T::kBytes,
                      "four O slices fit one K buffer");
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 pr;
                pr[0] = E::pack2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                pr[1] = E::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                const int c = 4 * db + g;
                *(LDS u32x2 *)(stage + l32 * T::kRowBytes + ((c ^ (l32 & (CH - 1))) << 4) +
                               8 * hh) = pr;
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int RPI = 64 / CH;                      // rows per store instruction
        constexpr int NIT = kRowsPerWave / RPI;
        const int rr = lane / CH, cc = lane % CH;
        u32x4 x[NIT];                                     // all reads first, then the stores
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = it * RPI + rr;
            x[it] = *(const LDS u32x4 *)(stage + r * T::kRowBytes + ((cc ^ (r & (CH - 1))) << 4));
        }
        const int rows_ok = (GEN ? len : N) - q0;         // valid rows of this wave's slab
        u16 *obase = O + head + (size_t)q0 * D + 8 * cc;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = it * RPI + rr;
            if (rows_ok >= kRowsPerWave || r < rows_ok)
                *(u32x4 *)(obase + (size_t)r * D) = x[it];
        }
        if ((GEN ? (qrow < len) : (qrow < N)) && hh == 0)
            LSE[row0 + qrow] = (m + log2f(lt)) * 0.69314718055994530942f;
    }
}

typedef void (*kernel_fn)(const u16 *, const u16 *, const u16 *, u16 *, float *,
                          int, int, int, float, unsigned, unsigned, int, int, int,
                          const int *, int, int, int, float *, float *, DropArgs);

template <int DT, int D>
kernel_fn pick_d(int mode, bool drop)
{
    if (drop) return mode == 1 ? fa_fwd_kernel<DT, D, 1, true> : fa_fwd_kernel<DT, D, 0, true>;
    switch (mode) {
    case 0: return fa_fwd_kernel<DT, D, 0, false>;
    case 1: return fa_fwd_kernel<DT, D, 1, false>;
    case 2: return fa_fwd_kernel<DT, D, 2, false>;
    case 3: return fa_fwd_kernel<DT, D, 3, false>;
    case 4: return fa_fwd_kernel<DT, D, 4, false>;
    default: return fa_fwd_kernel<DT, D, 5, false>;
    }
}

template <int DT>
kernel_fn pick(int d, int mode, bool drop)
{
    return d == 64 ? pick_d<DT, 64>(mode, drop) : pick_d<DT, 128>(mode, drop);
}

// Merge of the key segments of mode 3, per row ([P-baidu] §4.2-§4.3 and the
// split-K/V combination of "FlashAttention V2 核心原理与架构设计" §5.1):
// lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s, O rounded once.
// D / 4 lanes per row, 4 elements each.  Row i of a head (N rows) reads only
// the segments that hold one of its keys: with a right window side wr >= 0
// its keys end at i + wr, so segments 0 .. (i + wr) / kseg (each as wsp
// halves); the segments past them are never read (and may be unwritten).
constexpr int kMergeBatch = 16;   // segments whose loads the merge issues together

template <int DT, int D>
__global__ __launch_bounds__(256)
void fa_fwd_merge_kernel(const float *__restrict__ PO, const float *__restrict__ PL,
                         u16 *__restrict__ O, float *__restrict__ LSE, long long rows,
                         int nseg, int N, int kseg, int wr, int wsp)
{
    using E = Elem<DT>;
    constexpr int LPR = D / 4;
    constexpr int RPB = 256 / LPR;
    const long long r = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    if (r >= rows) return;
    const int nm = nseg * wsp;                         // partial slots per row
    int ns = nm;                                       // slots this row reads
    if (wr >= 0) {
        const long long last = (long long)(r % N) + wr;  // the row's last allowed key
        ns = (int)min((long long)nseg, last / kseg + 1) * wsp;
    }
    // segments in batches of kMergeBatch: each batch's lse and O slices are
    // requested at once, then merged into running sums kept against the
    // largest lse seen so far (rescaled when a batch raises it)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float sum = 0.f, mx = neg_inf();
    for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
        float ls[kMergeBatch];
        f32x4 x[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            ls[i] = neg_inf();
            if (s0 + i < ns) {
                const size_t sr = (size_t)(s0 + i) * rows + r;
                ls[i] = PL[sr];
                x[i] = *(const f32x4 *)(PO + sr * D + 4 * part);
            }
        }
        float bm = mx;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) bm = fmaxf(bm, ls[i]);
        if (bm == neg_inf()) continue;                // no key in any segment yet
        if (bm != mx) {
            const float a = (mx == neg_inf()) ? 0.f : __expf(mx - bm);
            sum *= a;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= a;
            mx = bm;
        }
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            if (ls[i] != neg_inf()) {
                const float wgt = __expf(ls[i] - mx);
                sum += wgt;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, x[i][e], acc[e]);
            }
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    u32x2 pr;
    pr[0] = E::pack2(acc[0] * inv, acc[1] * inv);
    pr[1] = E::pack2(acc[2] * inv, acc[3] * inv);
    *(u32x2 *)(O + r * D + 4 * part) = pr;
    if (part == 0) LSE[r] = sum > 0.f ? mx + logf(sum) : neg_inf();
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

namespace {

// Validation shared by every forward entry point, then one launch of the
// kernel for `mode` (0 full, 1 causal, 2 window / valid lengths).
fa_status validate_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int H, int N, int d, const int *lens, float scale,
                       fa_dtype dtype)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (N > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
        return FA_ERR_MISALIGNED;
    if (((uintptr_t)lse | (uintptr_t)lens) & 3) return FA_ERR_MISALIGNED;

    const long long BH = (long long)B * H;
    const long long nqb = (N + kBR - 1) / kBR;
    const long long grid = BH * nqb;
    if (BH > INT_MAX || grid > INT_MAX) return FA_ERR_INVALID_ARG;
    const size_t tbytes = (size_t)BH * (size_t)N * (size_t)d * 2;
    const size_t lbytes = (size_t)BH * (size_t)N * 4;
    if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
        overlaps(o, tbytes, v, tbytes) || overlaps(lse, lbytes, q, tbytes) ||
        overlaps(lse, lbytes, k, tbytes) || overlaps(lse, lbytes, v, tbytes) ||
        overlaps(lse, lbytes, o, tbytes))
        return FA_ERR_INVALID_ARG;
    if (lens && (overlaps(o, tbytes, lens, (size_t)B * 4) ||
                 overlaps(lse, lbytes, lens, (size_t)B * 4)))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

fa_status launch_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int H, int N, int d, int mode, int wl, int wr, const int *lens,
                     float scale, fa_dtype dtype, hipStream_t stream, int nseg = 1,
                     int kseg = 0, float *po = nullptr, float *pl = nullptr,
                     const DropArgs *drop = nullptr, int max_rows = 0, int nk = 0,
                     int wsplit = 1)
{
    // nk > 0 (mode 3 only): the rows run against nk keys per head, and the
    // caller has validated the differently sized tensors itself.  wsplit = 2
    // (mode 3, N <= 32 rows): two waves per work-group each compute half of
    // every key tile as segments of their own, so po / pl hold 2 * nseg
    // segments.
    if (mode < 4 && nk == 0) {
        const fa_status vs = validate_fwd(q, k, v, o, lse, B, H, N, d, lens, scale, dtype);
        if (vs != FA_OK) return vs;
    }
    const long long BH = (long long)B * H;
    const long long nqb = ((mode >= 4 ? max_rows : N) + kBR - 1) / kBR;
    const long long grid = BH * nqb;
    if (drop && mode > 1) return FA_ERR_INVALID_ARG;
    kernel_fn fn = (dtype == FA_DTYPE_F16) ? pick<FA_DTYPE_F16>(d, mode, drop != nullptr)
                                           : pick<FA_DTYPE_BF16>(d, mode, drop != nullptr);
    // Scores are always taken with a positive multiplier c: scale < 0 negates
    // Q exactly (sign bits) and scale == 0 zeroes Q (every score 0, every
    // allowed key weighted equally); c = |scale| log2(e), or log2(e) for 0.
    const float mag = (scale == 0.f) ? 1.f : fabsf(scale);
    float c = mag * 1.44269504088896340736f;
    unsigned qand = (scale == 0.f) ? 0u : 0xffffffffu;
    unsigned qxor = (scale < 0.f) ? 0x80008000u : 0u;
    int bh_i = (int)BH, n_i = N, nqb_i = (int)nqb, h_i = H, wl_i = wl, wr_i = wr;
    // the kernel splits a work-group's tiles over two waves only for mode 3
    // problems of at most one wave's rows; the merge then sees 2 * nseg
    const int wsp = (mode == 3 && wsplit > 1 && N <= kRowsPerWave) ? 2 : 1;
    const long long rows = BH * N;                    // merge rows (mode 3)
    const int rpb = 256 / (d / 4);
    const long long g2 = (rows + rpb - 1) / rpb;
    if (mode == 3 && g2 > INT_MAX) return FA_ERR_INVALID_ARG;
    int kseg_i = kseg, nk_i = nk > 0 ? nk : N, wsplit_i = wsp;
    const void *qp = q, *kp = k, *vp = v;
    void *op = o;
    float *lp = lse, *pop = po, *plp = pl;
    const int *lensp = lens;
    DropArgs dr = drop ? *drop : DropArgs{0u, 0u, 0u, 256u, 1.f};
    void *args[] = {&qp, &kp, &vp, &op, &lp, &bh_i, &n_i, &nqb_i, &c, &qand, &qxor,
                    &h_i, &wl_i, &wr_i, &lensp, &kseg_i, &nk_i, &wsplit_i, &pop, &plp, &dr};
    hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)grid, (unsigned)nseg),
                                   dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return FA_ERR_LAUNCH;
    if (mode == 3) {
        // the merge combines nseg * wsp partial slots per row, or fewer for
        // rows whose keys end early (wr >= 0)
        auto merge = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)g2), dim3(256), 0, stream, po, pl,
                               (u16 *)o, lse, rows, nseg, N, kseg, wr, wsp);
        };
        if (dtype == FA_DTYPE_F16) {
            if (d == 64) merge(fa_fwd_merge_kernel<FA_DTYPE_F16, 64>);
            else merge(fa_fwd_merge_kernel<FA_DTYPE_F16, 128>);
        } else {
            if (d == 64) merge(fa_fwd_merge_kernel<FA_DTYPE_BF16, 64>);
            else merge(fa_fwd_merge_kernel<FA_DTYPE_BF16, 128>);
        }
        if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
    }
    return FA_OK;
}

// Key segment length for num_splits requested splits: a whole number of
// LDS tiles; the number of non-empty segments can be smaller than asked.
int split_kseg(int N, int num_splits)
{
    const int per = (N + num_splits - 1) / num_splits;
    return ((per + kLT - 1) / kLT) * kLT;
}

}  // namespace

extern "C" fa_status fa_fwd(const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int H, int N, int d, int causal,
                            float scale, fa_dtype dtype, hipStream_t stream)
{
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    return launch_fwd(q, k, v, o, lse, B, H, N, d, causal, -1, causal ? 0 : -1, nullptr,
                      scale, dtype, stream);
}

extern "C" fa_status fa_fwd_window(const void *q, const void *k, const void *v, void *o,
                                   float *lse, int B, int H, int N, int d, int window_left,
                                   int window_right, const int *seqlens, float scale,
                                   fa_dtype dtype, hipStream_t stream)
{
    if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
    // a side of N or more allows every key on that side: clamp it to N so
    // the kernel's row +- side arithmetic stays far inside int
    if (N > 0) {
        window_left = window_left > N ? N : window_left;
        window_right = window_right > N ? N : window_right;
    }
    // the unwindowed and the causal case without lengths run the tuned kernels
    int mode = 2;
    if (!seqlens && window_left == -1 && window_right == -1) mode = 0;
    if (!seqlens && window_left == -1 && window_right == 0) mode = 1;
    return launch_fwd(q, k, v, o, lse, B, H, N, d, mode, window_left, window_right, seqlens,
                      scale, dtype, stream);
}

extern "C" size_t fa_fwd_split_workspace_size(int B, int H, int N, int d, int num_splits)
{
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || num_splits < 1 ||
        num_splits > FA_MAX_SPLITS)
        return 0;
    const int kseg = split_kseg(N, num_splits);
    const size_t nseg = (size_t)((N + kseg - 1) / kseg);
    return nseg * (size_t)B * (size_t)H * (size_t)N * (size_t)(d + 1) * sizeof(float);
}

extern "C" fa_status fa_fwd_split(const void *q, const void *k, const void *v, void *o,
                                  float *lse, int B, int H, int N, int d, int causal,
                                  float scale, int num_splits, float *ws, fa_dtype dtype,
                                  hipStream_t stream)
{
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS || !ws) return FA_ERR_INVALID_ARG;
    const fa_status vs = validate_fwd(q, k, v, o, lse, B, H, N, d, nullptr, scale, dtype);
    if (vs != FA_OK) return vs;
    if ((uintptr_t)ws & 15) return FA_ERR_MISALIGNED;
    const size_t wsb = fa_fwd_split_workspace_size(B, H, N, d, num_splits);
    const size_t tb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * 4;
    if (overlaps(ws, wsb, q, tb) || overlaps(ws, wsb, k, tb) || overlaps(ws, wsb, v, tb) ||
        overlaps(ws, wsb, o, tb) || overlaps(ws, wsb, lse, lb))
        return FA_ERR_INVALID_ARG;
    const int kseg = split_kseg(N, num_splits);
    const int nseg = (N + kseg - 1) / kseg;
    float *po = ws;
    float *pl = ws + (size_t)nseg * B * H * N * d;
    return launch_fwd(q, k, v, o, lse, B, H, N, d, 3, -1, causal ? 0 : -1, nullptr, scale,
                      dtype, stream, nseg, kseg, po, pl);
}

// Key segments for fa_fwd_decode's num_splits = 0: enough that the grid
// holds about one work-group per compute unit (256; a work-group takes most
// of a CU's LDS), with at least kMinSegTiles LDS tiles of keys per segment.
static constexpr int kMinSegTiles = 4;
static int decode_splits(int B, int H, int Nq, int Nk)
{
    const long long wg = (long long)B * H * ((Nq + kBR - 1) / kBR);
    long long ns = (256 + wg - 1) / wg;
    const long long by_keys = Nk / (kMinSegTiles * kLT);
    if (ns > by_keys) ns = by_keys;
    if (ns > FA_MAX_SPLITS) ns = FA_MAX_SPLITS;
    return ns < 1 ? 1 : (int)ns;
}

// Up to one wave's rows (32), two waves of each work-group compute alternate
// halves of every key tile, each half a segment of its own.
static int decode_wave_split(int Nq) { return Nq <= kRowsPerWave ? 2 : 1; }

extern "C" int fa_fwd_decode_splits(int B, int H, int Nq, int Nk)
{
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return 0;
    return decode_splits(B, H, Nq, Nk);
}

extern "C" size_t fa_fwd_decode_workspace_size(int B, int H, int Nq, int Nk, int d,
                                               int num_splits)
{
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128) || num_splits < 0 ||
        num_splits > FA_MAX_SPLITS)
        return 0;
    const int ns = num_splits ? num_splits : decode_splits(B, H, Nq, Nk);
    const int kseg = split_kseg(Nk, ns);
    const size_t nseg = (size_t)((Nk + kseg - 1) / kseg) * decode_wave_split(Nq);
    return nseg * (size_t)B * (size_t)H * (size_t)Nq * (size_t)(d + 1) * sizeof(float);
}

extern "C" fa_status fa_fwd_decode(const void *q, const void *k, const void *v, void *o,
                                   float *lse, int B, int H, int Nq, int Nk, int d, int causal,
                                   float scale, int num_splits, float *ws, fa_dtype dtype,
                                   hipStream_t stream)
{
    if (!q || !k || !v || !o || !lse || !ws) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
    if (num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (Nq > FA_MAX_N || Nk > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)ws) & 15)
        return FA_ERR_MISALIGNED;
    if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;
    const long long BH = (long long)B * H;
    const long long grid = BH * ((Nq + kBR - 1) / kBR);
    if (BH > INT_MAX || grid > INT_MAX) return FA_ERR_INVALID_ARG;
    const size_t qb = (size_t)BH * Nq * d * 2, kb = (size_t)BH * Nk * d * 2;
    const size_t lb = (size_t)BH * Nq * 4;
    const size_t wsb = fa_fwd_decode_workspace_size(B, H, Nq, Nk, d, num_splits);
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) ||
        overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
        overlaps(lse, lb, o, qb) || overlaps(ws, wsb, q, qb) || overlaps(ws, wsb, k, kb) ||
        overlaps(ws, wsb, v, kb) || overlaps(ws, wsb, o, qb) || overlaps(ws, wsb, lse, lb))
        return FA_ERR_INVALID_ARG;
    const int ns = num_splits ? num_splits : decode_splits(B, H, Nq, Nk);
    const int kseg = split_kseg(Nk, ns);
    const int nseg = (Nk + kseg - 1) / kseg;
    const int wsp = decode_wave_split(Nq);
    float *po = ws;
    float *pl = ws + (size_t)nseg * wsp * BH * Nq * d;
    // causal: the queries are the last Nq positions, so query i may use keys
    // up to i + Nk - Nq (a window right side of Nk - Nq >= 0)
    return launch_fwd(q, k, v, o, lse, B, H, Nq, d, 3, -1, causal ? Nk - Nq : -1, nullptr,
                      scale, dtype, stream, nseg, kseg, po, pl, nullptr, 0, Nk, wsp);
}

// Split partials of fa_fwd_split_noalloc: each device holds its own copy.
// Host code never passes this name to a kernel (on the host it is only a
// stand-in); it uses the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The address of `scratch` on device `dev`, which must be current; looked
// up on the first call for that device and kept.
hipError_t scratch_address(int dev, float **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = (float *)ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" fa_status fa_fwd_split_noalloc(const void *q, const void *k, const void *v,
                                          void *o, float *lse, int B, int H, int N, int d,
                                          int causal, float scale, int num_splits,
                                          fa_dtype dtype, hipStream_t stream)
{
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_INVALID_ARG;
    const fa_status vs = validate_fwd(q, k, v, o, lse, B, H, N, d, nullptr, scale, dtype);
    if (vs != FA_OK) return vs;
    if (fa_fwd_split_workspace_size(B, H, N, d, num_splits) > FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA_ERR_LAUNCH;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_LAUNCH;
        if (sdev != dev) return FA_ERR_INVALID_ARG;
    }
    float *ws = nullptr;
    if (scratch_address(dev, &ws) != hipSuccess) return FA_ERR_LAUNCH;
    const int kseg = split_kseg(N, num_splits);
    const int nseg = (N + kseg - 1) / kseg;
    float *po = ws;
    float *pl = ws + (size_t)nseg * B * H * N * d;
    return launch_fwd(q, k, v, o, lse, B, H, N, d, 3, -1, causal ? 0 : -1, nullptr, scale,
                      dtype, stream, nseg, kseg, po, pl);
}

extern "C" fa_status fa_fwd_dropout(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int H, int N, int d, int causal,
                                    float scale, float p_drop, unsigned long long seed,
                                    unsigned offset, fa_dtype dtype, hipStream_t stream)
{
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!(p_drop >= 0.f && p_drop < 1.f)) return FA_ERR_INVALID_ARG;
    const unsigned thr = (unsigned)floor((1.0 - (double)p_drop) * 256.0 + 0.5);
    const DropArgs dr = {(unsigned)seed, (unsigned)(seed >> 32), offset, thr,
                         thr ? 256.f / (float)thr : 0.f};
    return launch_fwd(q, k, v, o, lse, B, H, N, d, causal, -1, causal ? 0 : -1, nullptr, scale,
                      dtype, stream, 1, 0, nullptr, nullptr, &dr);
}

extern "C" fa_status fa_fwd_varlen(const void *q, const void *k, const void *v, void *o,
                                   float *lse, const int *cu_seqlens, int B, int H, int total,
                                   int max_seqlen, int d, int causal, float scale,
                                   fa_dtype dtype, hipStream_t stream)
{
    if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || total < 1 || max_seqlen < 1 || max_seqlen > total)
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (max_seqlen > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
        return FA_ERR_MISALIGNED;
    if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return FA_ERR_MISALIGNED;
    const long long BH = (long long)B * H;
    const long long grid = BH * ((max_seqlen + kBR - 1) / kBR);
    if (BH > INT_MAX || grid > INT_MAX) return FA_ERR_INVALID_ARG;
    const size_t tb = (size_t)H * (size_t)total * (size_t)d * 2;
    const size_t lb = (size_t)H * (size_t)total * 4, cb = ((size_t)B + 1) * 4;
    if (overlaps(o, tb, q, tb) || overlaps(o, tb, k, tb) || overlaps(o, tb, v, tb) ||
        overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, tb) || overlaps(lse, lb, v, tb) ||
        overlaps(lse, lb, o, tb) || overlaps(o, tb, cu_seqlens, cb) ||
        overlaps(lse, lb, cu_seqlens, cb))
        return FA_ERR_INVALID_ARG;
    return launch_fwd(q, k, v, o, lse, B, H, total, d, causal ? 5 : 4, -1, causal ? 0 : -1,
                      cu_seqlens, scale, dtype, stream, 1, 0, nullptr, nullptr, nullptr,
                      max_seqlen);
}

extern "C" fa_status fa_fwd_f16(const void *q, const void *k, const void *v, void *o,
                                float *lse, int B, int H, int N, int d, int causal,
                                float scale, hipStream_t stream)
{
    return fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, FA_DTYPE_F16, stream);
}

extern "C" fa_status fa_fwd_bf16(const void *q, const void *k, const void *v, void *o,
                                 float *lse, int B, int H, int N, int d, int causal,
                                 float scale, hipStream_t stream)
{
    return fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, FA_DTYPE_BF16, stream);
}

extern "C" const char *fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG:
        return "FA_ERR_INVALID_ARG: null pointer, non-positive size, causal not 0/1, "
               "non-finite scale, unknown dtype, overlapping buffers or grid too large";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128, N <= 2^22";
    case FA_ERR_MISALIGNED:
        return "FA_ERR_MISALIGNED: q/k/v/o need 16-byte alignment, lse 4-byte";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: HIP rejected the kernel launch";
    case FA_ERR_SCRATCH:
        return "FA_ERR_SCRATCH: the split partials exceed the static scratch "
               "(FA_NOALLOC_SCRATCH_BYTES); use fa_fwd_split with a workspace";
    default: return "unknown fa_status";
    }
}
