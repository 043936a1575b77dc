// fa_fwd.hip -- exact attention forward pass for MI355X (gfx950, CDNA4).
//
// Pages cited (by tag and section):
//   [P-notes] "FlashAttention v1 & v2 笔记"            (yiran529.github.io)
//   [P-baidu] "FlashAttention 优化原理与实现要点解析"    (cloud.baidu.com)
//   [P-wmrh]  "FlashAttention V2 核心原理与架构设计"     (wmrh.cn)
//
// What one work-group does.  The grid runs over (batch, head, Q-block)
// ([P-notes] §五.1: sequence-dimension parallelism).  A work-group owns BR
// query rows and loops over the K/V tiles with the Q block outer and the K/V
// block inner ([P-notes] §五.2, [P-wmrh] §2.2 "V2"), so its output tile is
// accumulated on chip and written once.  Each of its four wavefronts owns a
// 32-row slab of the queries ([P-notes] §五.3 split-Q): a wave's softmax
// statistics never leave the wave, and no cross-wave reduction exists.
//
// Per K/V tile, per wave ([P-baidu] §5, steps 1-4):
//   S^T = K_j Q_i^T                on MFMA 32x32x16 (16-bit in, fp32 acc)
//   mask (diagonal / ragged-tail tiles only)
//   m_new = max(m, rowmax(S) * c)      c = |scale| * log2(e)
//   alpha = 2^(m - m_new), P = 2^(S*c - m_new)
//   l = alpha * l + rowsum(P)          ([P-baidu] §4.2)
//   O^T = alpha * O^T + V_j^T P^T      on MFMA  ([P-baidu] §4.3)
// and after the last tile O = O / l, lse = (m + log2 l) * ln 2 ([P-baidu]
// §4.3 and §6: numerator and denominator are kept apart and divided once).
//
// Why S^T rather than S: with the 32x32 MFMA's output layout a lane holds 16
// key positions of ONE query column, and lanes l and l+32 hold the other 16.
// The row maximum is then a per-lane reduction plus one exchange between the
// two wave halves, the row sum needs no exchange until the end, and the fp32
// score registers, once rounded to 16 bits, are already the B operand of the
// P.V product -- no shuffles between the two MFMAs.
//
// K/V tiles pass through LDS, double buffered: tile j+1 is fetched from HBM
// into registers with 128-bit loads while tile j is computed, then written to
// the other LDS buffer.  K is stored [key][d] (its MFMA operand wants d
// contiguous); V is stored transposed [d][key] (the P.V operand wants keys
// contiguous).  Both rows are padded so the MFMA-operand reads of a wave hit
// distinct LDS banks.
//
// Causal tiles that lie wholly above the diagonal are never visited
// ([P-baidu] §7); the last Q block of a ragged N masks keys >= N and does not
// store rows >= N.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

#include "fa_fwd.h"

namespace {

typedef unsigned short u16;
typedef u16 u16x8 __attribute__((ext_vector_type(8)));
typedef u16 u16x4 __attribute__((ext_vector_type(4)));
typedef u16 u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 32 * kWaves;   // query rows per work-group
constexpr int kBC = 64;            // keys per K/V tile

// Element-type specifics: the MFMA and the fp32 -> 16-bit pair conversion
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
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Key position held by accumulator register r of a 32x32 MFMA output in
// wave half hh (lanes 32*hh .. 32*hh+31): rows 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(const u16 *__restrict__ Q, const u16 *__restrict__ K,
                   const u16 *__restrict__ V, u16 *__restrict__ O,
                   float *__restrict__ LSE, int BH, int N, int nqb, float c,
                   unsigned qsign)
{
    using E = Elem<DT>;
    constexpr int KP = D + 8;          // K row pitch in LDS (elements)
    constexpr int VP = kBC + 4;        // V^T row pitch in LDS (elements)
    constexpr int KSZ = kBC * KP;
    constexpr int VSZ = D * VP;
    constexpr int KT = D / 16;         // MFMA k-steps over d for S^T
    constexpr int DB = D / 32;         // 32-row blocks of O^T
    constexpr int CPR = D / 8;         // 16-byte chunks per row
    constexpr int NCH = kBC * CPR / kThreads;   // chunks per thread per tile
    static_assert(NCH == 2 || NCH == 4, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 smem[2 * (KSZ + VSZ)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // Work-group -> (batch*head, Q block).  Heads vary fastest so that, with
    // work-groups dealt round-robin over the 8 XCDs, every Q block of one head
    // lands on the same XCD (and L2) whenever B*H is a multiple of 8.  Causal
    // grids start with the longest (last) Q blocks.
    const int L = blockIdx.x;
    const int bh = L % BH;
    const int qb = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
    const size_t head = (size_t)bh * (size_t)N * D;
    const u16 *Qh = Q + head;
    const u16 *Kh = K + head;
    const u16 *Vh = V + head;

    const int q_first = qb * kBR + 32 * w;    // first query row of this wave
    const int qrow = q_first + l32;           // the query row of this lane
    const bool wave_live = q_first < N;

    // Q slab -> B-operand fragments, kept in registers for the whole loop.
    u16x8 qf[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
        if (qrow < N)
            x = *(const u16x8 *)(Qh + (size_t)qrow * D + 16 * kk + 8 * hh);
        qf[kk] = x ^ (u16)qsign;
    }

    const int kv_end = CAUSAL ? min(N, (qb + 1) * kBR) : N;
    const int n_tiles = (kv_end + kBC - 1) / kBC;

    // ---- K/V tile staging: HBM -> registers -> LDS
    u16x8 kreg[NCH], vreg[NCH];
    auto fetch = [&](int t) {
        const int kv0 = t * kBC;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci / CPR, col8 = ci % CPR;
            const int key = kv0 + row;
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (key < N) x = *(const u16x8 *)(Kh + (size_t)key * D + col8 * 8);
            kreg[i] = x;
        }
        const int col8 = tid % CPR, kg = tid / CPR;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int key = kv0 + kg * NCH + i;
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (key < N) x = *(const u16x8 *)(Vh + (size_t)key * D + col8 * 8);
            vreg[i] = x;
        }
    };
    auto stash = [&](int buf) {
        u16 *Ks = smem + buf * (KSZ + VSZ);
        u16 *Vs = Ks + KSZ;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci / CPR, col8 = ci % CPR;
            *(u16x8 *)(Ks + row * KP + col8 * 8) = kreg[i];
        }
        const int col8 = tid % CPR, kg = tid / CPR;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u16 *dst = Vs + (col8 * 8 + e) * VP + kg * NCH;
            if constexpr (NCH == 4) {
                u16x4 t = {vreg[0][e], vreg[1][e], vreg[2][e], vreg[3][e]};
                *(u16x4 *)dst = t;
            } else {
                u16x2 t = {vreg[0][e], vreg[1][e]};
                *(u16x2 *)dst = t;
            }
        }
    };

    fetch(0);
    stash(0);
    __syncthreads();

    float m_run = neg_inf();   // running max, log2 domain (scaled by c)
    float l_run = 0.f;         // this lane's half of the running sum
    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < n_tiles) fetch(t + 1);
        const u16 *Ks = smem + buf * (KSZ + VSZ);
        const u16 *Vs = Ks + KSZ;
        const int kv0 = t * kBC;
        const bool active = wave_live && (!CAUSAL || kv0 <= q_first + 31);
        if (active) {
            // S^T = K_j Q^T : two 32-key blocks
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KT; ++kk)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u16x8 kf =
                        *(const u16x8 *)(Ks + (32 * kb + l32) * KP + 16 * kk + 8 * hh);
                    s[kb] = E::mfma(kf, qf[kk], s[kb]);
                }

            const bool masked = (kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > q_first);
            if (masked) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + acc_row(r, hh);
                        const bool keep = key < N && (!CAUSAL || key <= qrow);
                        if (!keep) s[kb][r] = neg_inf();
                    }
            }

            // row maximum: in-lane, then across the two wave halves
            float mx = neg_inf();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = (mx == neg_inf()) ? neg_inf() : mx * c;
            const float m_new = fmaxf(m_run, mt);
            const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

            // P = 2^(S*c - m), rounded to 16 bits as the B operand of P.V
            u32x4 pk[kBC / 16];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_use));
                    float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, -m_use));
                    if (masked) {
                        p0 = (s[kb][r] == neg_inf()) ? 0.f : p0;
                        p1 = (s[kb][r + 1] == neg_inf()) ? 0.f : p1;
                    }
                    rs += p0 + p1;
                    pk[2 * kb + (r >> 3)][(r & 7) >> 1] = E::pack2(p0, p1);
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
            }

            // O^T += V_j^T P^T
#pragma unroll
            for (int kk = 0; kk < kBC / 16; ++kk) {
                const u16x8 pf = __builtin_bit_cast(u16x8, pk[kk]);
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const u16 *vp = Vs + (32 * b + l32) * VP + 16 * kk + 4 * hh;
                    const u16x4 lo = *(const u16x4 *)vp;
                    const u16x4 hi = *(const u16x4 *)(vp + 8);
                    const u16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[b] = E::mfma(vf, pf, oacc[b]);
                }
            }
        }
        if (t + 1 < n_tiles) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one division per row, 16-bit O, fp32 lse
    if (wave_live) {
        const float lt = l_run + __shfl_xor(l_run, 32);
        if (qrow < N) {
            const float inv = 1.f / lt;
            u16 *orow = O + head + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 pr;
                    pr[0] = E::pack2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
                    pr[1] = E::pack2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
                    *(u32x2 *)(orow + 32 * b + 8 * g + 4 * hh) = pr;
                }
            if (hh == 0)
                LSE[(size_t)bh * N + qrow] = (m_run + log2f(lt)) * 0.69314718055994530942f;
        }
    }
}

typedef void (*kernel_fn)(const u16 *, const u16 *, const u16 *, u16 *, float *,
                          int, int, int, float, unsigned);

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
    // scale < 0: negate Q exactly (flip its sign bits) and use |scale|, so the
    // running maximum is always taken over non-negatively scaled scores.
    const float c = fabsf(scale) * 1.44269504088896340736f;   // log2(e)
    const unsigned qsign = (scale < 0.f) ? 0x8000u : 0u;
    int bh_i = (int)BH, n_i = N, nqb_i = (int)nqb;
    float c_f = c;
    unsigned qs = qsign;
    const void *qp = q, *kp = k, *vp = v;
    void *op = o;
    float *lp = lse;
    void *args[] = {&qp, &kp, &vp, &op, &lp, &bh_i, &n_i, &nqb_i, &c_f, &qs};
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
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128, N <= 2^24";
    case FA_ERR_MISALIGNED:
        return "FA_ERR_MISALIGNED: q/k/v/o need 16-byte alignment, lse 4-byte";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: HIP rejected the kernel launch";
    default: return "unknown fa_status";
    }
}
