// fa_fwd.hip -- exact attention forward pass for MI355X (gfx950, CDNA4).
//
// Pages cited (by tag and section):
//   [P-notes] "FlashAttention v1 & v2 笔记"            (yiran529.github.io)
//   [P-baidu] "FlashAttention 优化原理与实现要点解析"    (cloud.baidu.com)
//   [P-wmrh]  "FlashAttention V2 核心原理与架构设计"     (wmrh.cn)
//
// Work decomposition.  The grid runs over (batch, head, Q block)
// ([P-notes] §五.1: parallelism along the sequence as well).  A work-group
// owns 128 query rows and walks the K/V tiles of 64 keys with the Q block
// outer and the K/V block inner ([P-notes] §五.2, [P-wmrh] §2.2 "V2"), so
// its output is accumulated on chip and written once.  Each of its four
// wavefronts owns a 32-row slab of the queries ([P-notes] §五.3, split-Q):
// softmax statistics never leave the wave and no cross-wave reduction exists.
//
// Per K/V tile j, per wave ([P-baidu] §5 steps 1-4, §4.2, §4.3):
//   S^T = K_j Q^T                 MFMA 32x32x16, 16-bit in, fp32 accumulate
//   mask                          diagonal and ragged-tail tiles only
//   m' = max(m, rowmax(S) c)      c = |scale| log2(e); log2 domain
//   P = 2^(S c - m'),  l = 2^(m - m') l + rowsum(P)
//   O^T = 2^(m - m') O^T + V_j^T P^T      MFMA, P rounded to 16 bits
// and after the last tile O = O / l, lse = (m + log2 l) ln 2 ([P-baidu] §4.3
// and §6: numerator and denominator kept apart, one division at the end).
//
// MI355X-specific choices (the pages' A100 design is prior art only):
//  * S^T rather than S.  In the 32x32 MFMA output a lane holds 16 keys of ONE
//    query column (lane l and l+32 share the column).  Row max and row sum are
//    per-lane work plus one v_permlane32_swap, and the fp32 scores, once
//    rounded to 16 bits, are already the B operand of the P.V product.
//  * Every accumulator lives in VGPRs (about 200 per lane), so two waves share
//    each SIMD (two work-groups per CU, each with its own barriers) and the
//    MFMA pipe of one wave overlaps the softmax VALU work of the other.
//    Measured on MI355X: a single wave that interleaves LDS operand reads
//    with its MFMAs sustains ~44 cycles per 32-cycle MFMA, two such waves per
//    SIMD ~37.5, so the MFMA work must come from two waves at once.  (Both an
//    in-wave software pipeline, S(j+1) on MFMA while P(j) is on VALU, and a
//    barrier-enforced A/B phase offset between the two waves of a SIMD
//    measured slower than letting two work-groups drift freely.)
//  * Reductions over a row (max, fp32 sum, rounded sum) run as short trees
//    or several independent chains, never one serial dependency chain.
//  * K/V tiles go HBM -> LDS with buffer_load ... lds (no registers, no VALU);
//    rows past N come back as zeros from the buffer range check.  K is read
//    with ds_read_b128, V with ds_read_b64_tr_b16, which delivers V^T
//    fragments directly.  16-byte chunks inside each row are XOR-swizzled so
//    both read patterns are bank-conflict free.
//  * The reference maximum m moves only when a tile's maximum exceeds it by
//    more than 8 (log2 units); then P <= 256 and the result is the same
//    quotient, while the O rescale (64 multiplies per lane) is almost never
//    executed.
//
// Causal K/V tiles wholly above the diagonal are never visited ([P-baidu]
// §7); the last Q block of a ragged N masks keys >= N and stores no rows >= N.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

#include "fa_fwd.h"

namespace {

typedef unsigned short u16;
typedef u16 u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;                 // one 32-column MFMA block
constexpr int kBR = kWaves * kRowsPerWave;       // query rows per work-group
constexpr int kBC = 64;                          // keys per K/V tile
constexpr float kLazy = 8.0f;                    // reference-max slack, log2 units
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

// Geometry of one K or V tile (kBC rows of D 16-bit elements) in LDS: rows
// are dense, 16-byte chunks inside a row are XOR-swizzled by a function of
// the row.  K rows: 16 consecutive rows reading one logical chunk (one
// ds_read_b128 per lane) land on distinct banks.  V rows: the 4 rows x 64
// bytes that 32 lanes of one transposing read touch land on distinct banks.
template <int D> struct Tile {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kChunks = D / 8;
    static constexpr int kBytes = kBC * kRowBytes;
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;
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

// Key (row) position held by accumulator register r of a 32x32 MFMA output
// in wave half hh: 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Value of x in the other half of the wave (lane l <-> l^32), via
// v_permlane32_swap: swap(x, x) yields [x_lo, x_lo] and [x_hi, x_hi].
__device__ __forceinline__ float half_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const u16 *__restrict__ Q, const u16 *__restrict__ K,
                   const u16 *__restrict__ V, u16 *__restrict__ O,
                   float *__restrict__ LSE, int BH, int N, int nqb, float c,
                   unsigned qand, unsigned qxor)
{
    using E = Elem<DT>;
    using T = Tile<D>;
    constexpr int KT = D / 16;    // MFMA k-steps over d
    constexpr int DB = D / 32;    // 32-row blocks of O^T
    constexpr int PT = kBC / 16;  // MFMA k-steps over the keys of a tile

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
    // wave index as a scalar: every per-wave decision below is a scalar branch
    const int w = (tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // Work-group -> (batch*head, Q block).  Heads vary fastest: with
    // work-groups dealt round-robin over the 8 XCDs, all Q blocks of one head
    // share an XCD (and its L2) whenever B*H is a multiple of 8.  Causal
    // grids start with the longest (last) Q blocks.
    const int L = blockIdx.x;
    const int bh = L % BH;
    const int qblk = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
    const size_t head = (size_t)bh * (size_t)N * D;
    const int nbytes = N * T::kRowBytes;
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void *)(Q + head), 0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)(K + head), 0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void *)(V + head), 0, nbytes, kRsrcWord3);

    const int q0 = qblk * kBR + kRowsPerWave * w;   // first query row of this wave
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

    const int n_keys_tiles = (N + kBC - 1) / kBC;
    const int n_tiles = CAUSAL ? min(n_keys_tiles, (qblk + 1) * (kBR / kBC)) : n_keys_tiles;
    // tiles this wave computes: causal rows q0..q0+31 need keys <= q0+31
    const int n_w = (q0 >= N) ? 0 : (CAUSAL ? min(n_tiles, (q0 + kRowsPerWave - 1) / kBC + 1)
                                            : n_tiles);

    // ---- HBM -> LDS tile loads (each wave moves its share, 1 KB per load)
    auto issue = [&](const __amdgpu_buffer_rsrc_t &r, auto buf, int t) {
        constexpr bool is_v = decltype(buf)::value >= 2;
#pragma unroll
        for (int j = 0; j < T::kLoadsPerWave; ++j) {
            const int li = w * T::kLoadsPerWave + j;
            const int row = li * T::kRowsPerLoad + lane / T::kChunks;
            const int pc = lane % T::kChunks;
            const int lc = pc ^ (is_v ? T::vswz(row) : T::kswz(row));
            const int off = (t * kBC + row) * T::kRowBytes + lc * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (LDS void *)(bufp(buf) + li * 1024), 16, off, 0, 0, 0);
        }
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

    auto kfrag = [&](auto buf, int kb, int kk) -> u16x8 {
        return *(const LDS u16x8 *)(bufp(buf) + kb * 32 * T::kRowBytes + koff[kk]);
    };
    auto vfrag = [&](auto buf, int db, int kk) -> u16x8 {
        const LDS unsigned char *p = bufp(buf) + kk * 16 * T::kRowBytes + voff[db];
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4 *)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS s16x4 *)(p + 8 * T::kRowBytes));
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // S^T(j) = K_j Q^T: s[kb], keys 32*kb.., query column l32.  Operands
    // are read from LDS kDepth k-steps ahead of their MFMAs.
    constexpr int kDepth = 2;
    auto qk = [&](f32x16 (&s)[2], auto buf) {
        u16x8 kf[kDepth + 1][2];
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            kf[i][0] = kfrag(buf, 0, i);
            kf[i][1] = kfrag(buf, 1, i);
        }
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            if (kk + kDepth < KT) {
                kf[(kk + kDepth) % (kDepth + 1)][0] = kfrag(buf, 0, kk + kDepth);
                kf[(kk + kDepth) % (kDepth + 1)][1] = kfrag(buf, 1, kk + kDepth);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u16x8 a = kf[kk % (kDepth + 1)][kb];
                if (kk == 0) {
                    const f32x16 z = {};
                    s[kb] = E::mfma(a, qf[kk], z);
                } else {
                    s[kb] = E::mfma(a, qf[kk], s[kb]);
                }
            }
        }
    };

    auto mask = [&](f32x16 (&s)[2], int t) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t * kBC + 32 * kb + acc_row(r, hh);
                const bool keep = key < N && (!CAUSAL || key <= qrow);
                if (!keep) s[kb][r] = neg_inf();
            }
    };

    float m = neg_inf();   // reference max, log2 domain
    float l = 0.f;         // this lane's half of the row sum of P (fp32)
    float lh = 0.f;        // the same sum of P rounded to 16 bits
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

    // Row max of S(j) and the (lazy) update of the reference max.
    auto update_max = [&](f32x16 (&s)[2]) {
        // 32 values -> 11 -> 4 -> 1 with three-input maxima (depth 4)
        float t1[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            const int a = 3 * i, b = 3 * i + 1, e = 3 * i + 2;
            t1[i] = fmaxf(fmaxf(s[a >> 4][a & 15], s[b >> 4][b & 15]), s[e >> 4][e & 15]);
        }
        t1[10] = fmaxf(s[1][14], s[1][15]);
        const float u0 = fmaxf(fmaxf(t1[0], t1[1]), t1[2]);
        const float u1 = fmaxf(fmaxf(t1[3], t1[4]), t1[5]);
        const float u2 = fmaxf(fmaxf(t1[6], t1[7]), t1[8]);
        const float u3 = fmaxf(t1[9], t1[10]);
        const float mx = fmaxf(fmaxf(fmaxf(u0, u1), u2), u3);
        const float mt = half_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mt > m + kLazy)) {
            const float mn = fmaxf(m, mt);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m - mu);
            if constexpr (DT == FA_DTYPE_BF16) l *= alpha;
            lh *= alpha;
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
    auto softmax = [&](f32x16 (&s)[2], u32x4 (&pk)[PT]) {
        const float mu = (m == neg_inf()) ? 0.f : m;
        float rs[4], rh[4];
        // groups of 8 scores: 8 FMAs, 8 exps, then sums and packing, so the
        // temporaries die inside the group (scheduling barrier per group)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int kb = g >> 1, r0 = (g & 1) * 8;
            float x[8], p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = fmaf(s[kb][r0 + e], c, -mu);
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(x[e]);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (DT == FA_DTYPE_BF16) {
                    const float a = p[2 * h] + p[2 * h + 1];
                    rs[h] = (g == 0) ? a : rs[h] + a;
                }
                const unsigned pr = E::pack2(p[2 * h], p[2 * h + 1]);
                rh[h] = E::sum2(pr, (g == 0) ? 0.f : rh[h]);
                pk[2 * kb + (r0 >> 3)][h] = pr;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DT == FA_DTYPE_BF16) l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        lh += (rh[0] + rh[1]) + (rh[2] + rh[3]);
    };

    // O^T += V_j^T P(j)^T, operands prefetched 2*kDepth MFMAs ahead
    auto pv = [&](auto buf, u32x4 (&pk)[PT]) {
        constexpr int NM = PT * DB;        // MFMAs, index i -> kk = i / DB, db = i % DB
        constexpr int AHEAD = 2 * kDepth;
        u16x8 vf[AHEAD + 1];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) vf[i] = vfrag(buf, i % DB, i / DB);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i + AHEAD < NM)
                vf[(i + AHEAD) % (AHEAD + 1)] = vfrag(buf, (i + AHEAD) % DB, (i + AHEAD) / DB);
            oacc[i % DB] = E::mfma(vf[i % (AHEAD + 1)],
                                   __builtin_bit_cast(u16x8, pk[i / DB]), oacc[i % DB]);
        }
    };

    auto tile_masked = [&](int t) {
        const bool mk = (CAUSAL && t * kBC + kBC - 1 > q0) || (t * kBC + kBC > N);
        return __builtin_amdgcn_readfirstlane((int)mk) != 0;
    };

    // ---- prologue: K_0, V_0, K_1 in flight; S(0)
    issue(rk, Buf<0>{}, 0);
    issue(rv, Buf<2>{}, 0);
    if (n_tiles > 1) issue(rk, Buf<1>{}, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 sA[2], sB[2];
    if (n_w > 0) {
        qk(sA, Buf<0>{});
        if (tile_masked(0)) mask(sA, 0);
        update_max(sA);
    }
    __syncthreads();   // K_0 fully consumed before K_2 overwrites buffer 0

    // One tile step (t has parity P): P(t) from scur, O += V_t P(t), then
    // S(t+1) into snext; meanwhile K_{t+2} and V_{t+1} stream into the
    // buffers that step t-1 finished with.
    auto step = [&](auto par, int t, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
        constexpr int P = decltype(par)::value;
        if (t + 2 < n_tiles) issue(rk, Buf<P>{}, t + 2);
        if (t + 1 < n_tiles) issue(rv, Buf<3 - P>{}, t + 1);
        if (t < n_w) {
            u32x4 pk[PT];
            if (t + 1 < n_w) {
                softmax(scur, pk);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(2);
                pv(Buf<2 + P>{}, pk);
                __builtin_amdgcn_sched_barrier(0);
                qk(snext, Buf<1 - P>{});
                __builtin_amdgcn_s_setprio(0);
                if (tile_masked(t + 1)) mask(snext, t + 1);
                update_max(snext);
            } else {
                softmax(scur, pk);
                pv(Buf<2 + P>{}, pk);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    for (int t = 0; t < n_tiles; t += 2) {
        step(Buf<0>{}, t, sA, sB);
        if (t + 1 < n_tiles) step(Buf<1>{}, t + 1, sB, sA);
    }

    // ---- epilogue: one division per row, 16-bit O, fp32 lse
    if (n_w > 0) {
        const float lht = half_sum(lh);
        const float lt = (DT == FA_DTYPE_BF16) ? half_sum(l) : lht;
        if (qrow < N) {
            const float inv = 1.f / lht;
            u16 *orow = O + head + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 pr;
                    pr[0] = E::pack2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                    pr[1] = E::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                    *(u32x2 *)(orow + 32 * db + 8 * g + 4 * hh) = pr;
                }
            if (hh == 0)
                LSE[(size_t)bh * N + qrow] = (m + log2f(lt)) * 0.69314718055994530942f;
        }
    }
}

typedef void (*kernel_fn)(const u16 *, const u16 *, const u16 *, u16 *, float *,
                          int, int, int, float, unsigned, unsigned);

template <int DT>
kernel_fn pick(int d, int causal)
{
    if (d == 64) return causal ? fa_fwd_kernel<DT, 64, true> : fa_fwd_kernel<DT, 64, false>;
    return causal ? fa_fwd_kernel<DT, 128, true> : fa_fwd_kernel<DT, 128, false>;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" fa_status fa_fwd(const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int H, int N, int d, int causal,
                            float scale, fa_dtype dtype, hipStream_t stream)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (N > FA_MAX_N) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
        return FA_ERR_MISALIGNED;
    if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;

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

    kernel_fn fn = (dtype == FA_DTYPE_F16) ? pick<FA_DTYPE_F16>(d, causal)
                                           : pick<FA_DTYPE_BF16>(d, causal);
    // Scores are always taken with a positive multiplier c: scale < 0 negates
    // Q exactly (sign bits) and scale == 0 zeroes Q (every score 0, every
    // allowed key weighted equally); c = |scale| log2(e), or log2(e) for 0.
    const float mag = (scale == 0.f) ? 1.f : fabsf(scale);
    float c = mag * 1.44269504088896340736f;
    unsigned qand = (scale == 0.f) ? 0u : 0xffffffffu;
    unsigned qxor = (scale < 0.f) ? 0x80008000u : 0u;
    int bh_i = (int)BH, n_i = N, nqb_i = (int)nqb;
    const void *qp = q, *kp = k, *vp = v;
    void *op = o;
    float *lp = lse;
    void *args[] = {&qp, &kp, &vp, &op, &lp, &bh_i, &n_i, &nqb_i, &c, &qand, &qxor};
    hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)grid), dim3(kThreads),
                                   args, 0, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
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
    default: return "unknown fa_status";
    }
}
