/*
 * oracle.c -- plain, slow, fp64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library: it has its own 16-bit decoders and its own loops.
 *
 * Sources (web pages; cited by tag and section):
 *   [P-notes] "FlashAttention v1 & v2 笔记"              (yiran529.github.io)
 *   [P-baidu] "FlashAttention 优化原理与实现要点解析"      (cloud.baidu.com)
 *   [P-wmrh]  "FlashAttention V2 核心原理与架构设计"       (wmrh.cn)
 *
 * What is computed (per batch b, head h, query row i):
 *   A_i   = {0..N-1}, or {0..i} when causal (key j <= query i);
 *   s_j   = scale * sum_c q[i][c] * k[j][c]                  for j in A_i
 *   o[i]  = sum_j softmax(s)_j * v[j]
 *   lse_i = ln sum_{j in A_i} exp(s_j)
 * i.e. Attention(Q,K,V) = Softmax(Q K^T * scale) V, [P-baidu] §1 (the formula)
 * and §2 (S = QK^T, P = Softmax(S), O = PV).  The softmax is the max-shifted
 * form of [P-baidu] §4.1 (max pass, then exp-sum, then normalise).  The
 * logsumexp output packs the row maximum m and denominator l that the kernel
 * signature in [P-wmrh] §2.3 returns separately: lse = m + ln l.
 *
 * Tensors are [B,H,N,d] contiguous, element (b,h,n,c) at ((b*H+h)*N+n)*d+c.
 * Inputs are raw IEEE binary16 (dtype 0) or bfloat16 (dtype 1) bit patterns.
 *
 * The tiled function oracle_attn_fwd_tiled() follows the block algorithm of
 * [P-baidu] §4.2, §4.3, §5 and §6 step by step in fp64; it exists so that the
 * merge algebra can be checked against the plain definition.
 *
 * Parity pins (all in the CPU test suite): brute force against a library
 * softmax on tiny inputs, rows of P summing to 1, constant-V, identical-K,
 * Q = 0, causal row 0, shift and permutation invariance, the tiled merge at
 * several tile sizes, peaky inputs, and exhaustive decoder checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DTYPE_F16 0
#define ORACLE_DTYPE_BF16 1

/* ---- 16-bit decoders ---------------------------------------------------- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * Subnormals (exponent 0) are fraction * 2^-24. */
static double decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = (f == 0) ? INFINITY : NAN;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 * Subnormals (exponent 0) are fraction * 2^-133. */
static double decode_bf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133);
    else if (e == 255)
        mag = (f == 0) ? INFINITY : NAN;
    else
        mag = ldexp((double)(128 + f), e - 134);
    return sign ? -mag : mag;
}

static int decode_all(const uint16_t *bits, int dtype, int64_t n, double *out)
{
    if (dtype == ORACLE_DTYPE_F16) {
        for (int64_t i = 0; i < n; ++i) out[i] = decode_f16(bits[i]);
    } else if (dtype == ORACLE_DTYPE_BF16) {
        for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16(bits[i]);
    } else {
        return -1;
    }
    return 0;
}

int oracle_decode(const uint16_t *bits, int dtype, int64_t n, double *out)
{
    return decode_all(bits, dtype, n, out);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- 1-D softmax, two ways --------------------------------------------- */

/* [P-baidu] §4.1: pass 1 finds the maximum m, pass 2 sums exp(x_j - m),
 * pass 3 normalises each element. */
void oracle_softmax_1d(const double *x, int64_t n, double *out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (x[j] > m) m = x[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) l += exp(x[j] - m);
    for (int64_t j = 0; j < n; ++j) out[j] = exp(x[j] - m) / l;
}

/* [P-wmrh] §2.1: one pass keeping a running maximum m and a running sum l;
 * each new element first rescales l by exp(m - m_new), then adds
 * exp(x_i - m_new).  Result exp(x - m) / l.  (The page's code lost its '='
 * and '+' signs in extraction; this is the recurrence it describes.) */
void oracle_softmax_online_1d(const double *x, int64_t n, double *out)
{
    double m = -INFINITY, l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double m_new = x[i] > m ? x[i] : m;
        /* Boundary cases (§2.1 asks for them to be handled): while every
         * element so far is -inf, m = -inf and l = 0; a -inf element adds
         * weight 0 (exp(-inf - (-inf)) would be NaN). */
        double scale_old = (m == -INFINITY) ? 0.0 : exp(m - m_new);
        double term = (x[i] == -INFINITY) ? 0.0 : exp(x[i] - m_new);
        l = l * scale_old + term;
        m = m_new;
    }
    for (int64_t j = 0; j < n; ++j) out[j] = exp(x[j] - m) / l;
}

/* ---- exact attention, plain definition ---------------------------------- */

typedef struct {
    double *q, *k, *v;          /* decoded [B,H,N,d] */
    int64_t B, H, N, d;
    int causal;
    double scale;
} problem;

static int load_problem(problem *p, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, int dtype, int64_t B, int64_t H,
                        int64_t N, int64_t d, int causal, double scale)
{
    if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
    if (dtype != ORACLE_DTYPE_F16 && dtype != ORACLE_DTYPE_BF16) return -1;
    int64_t n = B * H * N * d;
    p->B = B; p->H = H; p->N = N; p->d = d; p->causal = causal; p->scale = scale;
    size_t bytes = (size_t)(n > 0 ? n : 1) * sizeof(double);
    p->q = (double *)malloc(bytes);
    p->k = (double *)malloc(bytes);
    p->v = (double *)malloc(bytes);
    if (!p->q || !p->k || !p->v) {
        free(p->q); free(p->k); free(p->v);
        return -2;
    }
    decode_all(q, dtype, n, p->q);
    decode_all(k, dtype, n, p->k);
    decode_all(v, dtype, n, p->v);
    return 0;
}

static void free_problem(problem *p)
{
    free(p->q); free(p->k); free(p->v);
}

/* One query row.  `row` is the flat index (b*H+h)*N+i.  `s` is scratch of
 * N doubles.  Writes d values to o_out and one to lse_out. */
static void attn_row(const problem *p, int64_t row, double *s, double *o_out,
                     double *lse_out)
{
    const int64_t N = p->N, d = p->d;
    const int64_t bh = row / N, i = row % N;
    const double *qi = p->q + row * d;
    const double *kh = p->k + bh * N * d;
    const double *vh = p->v + bh * N * d;
    const int64_t nkeys = p->causal ? i + 1 : N;     /* |A_i| */

    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
        s[j] = p->scale * dot;
        if (s[j] > m) m = s[j];
    }
    /* pass 2: weights, denominator, weighted sum of V */
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o_out[c] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        double w = exp(s[j] - m);
        l += w;
        for (int64_t c = 0; c < d; ++c) o_out[c] += w * vh[j * d + c];
    }
    /* normalise */
    for (int64_t c = 0; c < d; ++c) o_out[c] /= l;
    *lse_out = m + log(l);
}

/* Full forward: o is [B,H,N,d] fp64, lse is [B,H,N] fp64. */
int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                    int causal, double scale, double *o, double *lse)
{
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r)
                attn_row(&p, r, s, o + r * d, lse + r);
        }
        free(s);
    }
    free_problem(&p);
    return fail ? -2 : 0;
}

/* Selected rows only: rows[t] is a flat row index (b*H+h)*N+i; outputs are
 * packed, o_rows is [n_rows, d] and lse_rows is [n_rows]. */
int oracle_attn_fwd_rows(const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, int dtype, int64_t B, int64_t H,
                         int64_t N, int64_t d, int causal, double scale,
                         const int64_t *rows, int64_t n_rows, double *o_rows,
                         double *lse_rows)
{
    const int64_t total = B * H * N;
    for (int64_t t = 0; t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= total) return -1;
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < n_rows; ++t)
                attn_row(&p, rows[t], s, o_rows + t * d, lse_rows + t);
        }
        free(s);
    }
    free_problem(&p);
    return fail ? -2 : 0;
}

/* The attention weights P = Softmax(S) themselves, [B,H,N,N] fp64, masked
 * entries 0.  For tiny inputs only ([P-baidu] §2 step 2). */
int oracle_attn_probs(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                      int causal, double scale, double *probs)
{
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!s) { free_problem(&p); return -2; }
    for (int64_t r = 0; r < B * H * N; ++r) {
        const int64_t bh = r / N, i = r % N;
        const int64_t nkeys = causal ? i + 1 : N;
        double *prow = probs + r * N;
        for (int64_t j = 0; j < N; ++j) prow[j] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dot += p.q[r * d + c] * p.k[(bh * N + j) * d + c];
            s[j] = scale * dot;
        }
        oracle_softmax_1d(s, nkeys, prow);
    }
    free(s);
    free_problem(&p);
    return 0;
}

/* ---- the block algorithm, in fp64 ---------------------------------------
 *
 * [P-baidu] §5: Q is split into blocks of Br rows (outer loop) and K/V into
 * blocks of Bc rows (inner loop).  For each (Q block, K/V block):
 *   1. the score block S_blk = Q_blk K_blk^T * scale;
 *   2. per row, the block's local maximum m_new and local exponent sum
 *      l_new = sum exp(s - m_new), and (§6) the block's local numerator
 *      u_new = sum exp(s - m_new) v  -- numerator and denominator kept apart;
 *   3. the running maximum m = max(m_old, m_new) and (§4.2)
 *      l = l_old * exp(m_old - m) + l_new * exp(m_new - m);
 *   4. (§4.3) the running output O = O_old * exp(m_old - m)
 *      + u_new * exp(m_new - m), i.e. P_new V_new with P_new = exp(S - m);
 *   5. repeat over the K/V blocks;
 *   6. O_final = O / l  (§4.3, §6: one division at the end).
 * Rows whose allowed keys miss a block entirely (causal) skip that block;
 * [P-baidu] §7 notes whole blocks past the diagonal need no work.
 * Br = Bc = 1 reduces to the per-element recurrence of [P-wmrh] §2.1.
 */
int oracle_attn_fwd_tiled(const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, int dtype, int64_t B, int64_t H,
                          int64_t N, int64_t d, int causal, double scale,
                          int64_t Br, int64_t Bc, double *o, double *lse)
{
    if (Br < 1 || Bc < 1) return -1;
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    double *m = (double *)malloc((size_t)Br * sizeof(double));
    double *l = (double *)malloc((size_t)Br * sizeof(double));
    double *acc = (double *)malloc((size_t)(Br * d) * sizeof(double));
    double *sblk = (double *)malloc((size_t)(Br * Bc) * sizeof(double));
    double *unew = (double *)malloc((size_t)d * sizeof(double));
    if (!m || !l || !acc || !sblk || !unew) {
        free(m); free(l); free(acc); free(sblk); free(unew);
        free_problem(&p);
        return -2;
    }
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double *qh = p.q + bh * N * d;
        const double *kh = p.k + bh * N * d;
        const double *vh = p.v + bh * N * d;
        for (int64_t i0 = 0; i0 < N; i0 += Br) {           /* Q blocks: outer */
            const int64_t br = (N - i0 < Br) ? N - i0 : Br;
            for (int64_t r = 0; r < br; ++r) {
                m[r] = -INFINITY;
                l[r] = 0.0;
                for (int64_t c = 0; c < d; ++c) acc[r * d + c] = 0.0;
            }
            for (int64_t j0 = 0; j0 < N; j0 += Bc) {       /* K/V blocks: inner */
                const int64_t bc = (N - j0 < Bc) ? N - j0 : Bc;
                /* step 1: score block, masked entries -inf */
                for (int64_t r = 0; r < br; ++r)
                    for (int64_t t = 0; t < bc; ++t) {
                        const int64_t i = i0 + r, j = j0 + t;
                        if (causal && j > i) {
                            sblk[r * Bc + t] = -INFINITY;
                            continue;
                        }
                        double dot = 0.0;
                        for (int64_t c = 0; c < d; ++c)
                            dot += qh[i * d + c] * kh[j * d + c];
                        sblk[r * Bc + t] = scale * dot;
                    }
                for (int64_t r = 0; r < br; ++r) {
                    const double *srow = sblk + r * Bc;
                    /* step 2: local maximum, local denominator and numerator */
                    double m_new = -INFINITY;
                    for (int64_t t = 0; t < bc; ++t)
                        if (srow[t] > m_new) m_new = srow[t];
                    if (m_new == -INFINITY) continue;   /* no allowed key here */
                    double l_new = 0.0;
                    for (int64_t c = 0; c < d; ++c) unew[c] = 0.0;
                    for (int64_t t = 0; t < bc; ++t) {
                        double w = exp(srow[t] - m_new);   /* 0 for masked */
                        l_new += w;
                        for (int64_t c = 0; c < d; ++c)
                            unew[c] += w * vh[(j0 + t) * d + c];
                    }
                    /* step 3: merge the statistics */
                    const double m_old = m[r];
                    const double mm = m_old > m_new ? m_old : m_new;
                    const double f_old = (m_old == -INFINITY) ? 0.0 : exp(m_old - mm);
                    const double f_new = exp(m_new - mm);
                    l[r] = l[r] * f_old + l_new * f_new;
                    /* step 4: rescale the old numerator, add the new one */
                    for (int64_t c = 0; c < d; ++c)
                        acc[r * d + c] = acc[r * d + c] * f_old + unew[c] * f_new;
                    m[r] = mm;
                }
            }
            /* step 6: one division per row at the end */
            for (int64_t r = 0; r < br; ++r) {
                const int64_t row = bh * N + i0 + r;
                for (int64_t c = 0; c < d; ++c)
                    o[row * d + c] = acc[r * d + c] / l[r];
                lse[row] = m[r] + log(l[r]);
            }
        }
    }
    free(m); free(l); free(acc); free(sblk); free(unew);
    free_problem(&p);
    return 0;
}

/* ---- gradients of the plain definition ------------------------------------
 *
 * The pages state that the forward pass keeps the per-row statistics (the
 * maximum and the denominator, here packed as lse) so that the backward pass
 * can use them ([P-baidu] §6, "numerator and denominator kept apart", and the
 * V1/V2 comparison of §7; [P-wmrh] §2.3 outputs l and m), but print no
 * gradient formulas.  This is the gradient of the forward definition above,
 * obtained by the chain rule, for an upstream gradient dO of O:
 *
 *   P_ij  = softmax_j(s_i)               (j in A_i, 0 elsewhere)
 *   dV_j  = sum_i P_ij dO_i              (O = P V)
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - sum_t P_it dP_it)      (Jacobian of the softmax)
 *   dQ_i  = scale * sum_j dS_ij k_j      (s_ij = scale q_i . k_j)
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * fp64 throughout; dO is a 16-bit input like q, k, v.  All outputs fp64.
 *
 * The row term sum_t P_it dP_it equals dO_i . O_i, because O_i =
 * sum_t P_it v_t.  A backward pass that is handed the forward's 16-bit
 * output o uses D_i = dO_i . o_i instead; passing o (16-bit bits, or NULL)
 * selects that form, which differs from the plain one only through the
 * rounding of o.
 */

typedef struct {
    problem p;
    double *dO;
    double *o;          /* decoded given output, or NULL */
} bproblem;

static int load_bproblem(bproblem *bp, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const uint16_t *dO, const uint16_t *o,
                         int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                         int causal, double scale)
{
    int rc = load_problem(&bp->p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    int64_t n = B * H * N * d;
    bp->dO = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    bp->o = o ? (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)) : NULL;
    if (!bp->dO || (o && !bp->o)) {
        free(bp->dO); free(bp->o); free_problem(&bp->p);
        return -2;
    }
    decode_all(dO, dtype, n, bp->dO);
    if (o) decode_all(o, dtype, n, bp->o);
    return 0;
}

static void free_bproblem(bproblem *bp)
{
    free_problem(&bp->p);
    free(bp->dO);
    free(bp->o);
}

/* Row i of head bh: P_i. (into prow, nkeys entries), dP_i. (into dprow) and
 * returns D_i = sum_t P_it dP_it (or dO_i . o_i when o is given);
 * *lse_out (if not NULL) = ln sum_t exp(s_it). */
static double grad_row(const bproblem *bp, int64_t bh, int64_t i, double *prow,
                       double *dprow, double *lse_out)
{
    const problem *p = &bp->p;
    const int64_t N = p->N, d = p->d;
    const double *qi = p->q + (bh * N + i) * d;
    const double *doi = bp->dO + (bh * N + i) * d;
    const double *kh = p->k + bh * N * d;
    const double *vh = p->v + bh * N * d;
    const int64_t nkeys = p->causal ? i + 1 : N;
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
        prow[j] = p->scale * dot;
        if (prow[j] > m) m = prow[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        prow[j] = exp(prow[j] - m);
        l += prow[j];
    }
    if (lse_out) *lse_out = m + log(l);
    double D = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        prow[j] /= l;
        double dp = 0.0;
        for (int64_t c = 0; c < d; ++c) dp += doi[c] * vh[j * d + c];
        dprow[j] = dp;
        D += prow[j] * dp;
    }
    if (bp->o) {
        const double *oi = bp->o + (bh * N + i) * d;
        D = 0.0;
        for (int64_t c = 0; c < d; ++c) D += doi[c] * oi[c];
    }
    return D;
}

/* Full gradients: dq, dk, dv are [B,H,N,d] fp64.  Heads run in parallel;
 * within a head the rows run in order (dk and dv sum over rows). */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const uint16_t *dO, const uint16_t *o, int dtype, int64_t B,
                    int64_t H, int64_t N, int64_t d, int causal, double scale,
                    double *dq, double *dk, double *dv)
{
    bproblem bp;
    int rc = load_bproblem(&bp, q, k, v, dO, o, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    const int64_t n = B * H * N * d;
    for (int64_t t = 0; t < n; ++t) dq[t] = dk[t] = dv[t] = 0.0;
    int fail = 0;
#pragma omp parallel
    {
        double *prow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *dprow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!prow || !dprow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                const double *qh = bp.p.q + bh * N * d, *kh = bp.p.k + bh * N * d;
                const double *doh = bp.dO + bh * N * d;
                double *dqh = dq + bh * N * d, *dkh = dk + bh * N * d, *dvh = dv + bh * N * d;
                for (int64_t i = 0; i < N; ++i) {
                    const double D = grad_row(&bp, bh, i, prow, dprow, NULL);
                    const int64_t nkeys = causal ? i + 1 : N;
                    for (int64_t j = 0; j < nkeys; ++j) {
                        const double ds = prow[j] * (dprow[j] - D);
                        for (int64_t c = 0; c < d; ++c) {
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qh[i * d + c];
                            dvh[j * d + c] += prow[j] * doh[i * d + c];
                        }
                    }
                }
            }
        }
        free(prow);
        free(dprow);
    }
    free_bproblem(&bp);
    return fail ? -2 : 0;
}

/* Sampled gradients for inputs too large for oracle_attn_bwd: dq for the
 * flat query rows qrows[] ((b*H+h)*N+i) and dk, dv for the flat key rows
 * krows[] ((b*H+h)*N+j); outputs packed [n_q,d] and [n_k,d].  A key row
 * needs P_ij and D_i of every query row of its head, so those heads' rows
 * are evaluated once first (lse_i and D_i kept per row). */
int oracle_attn_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *dO, const uint16_t *o, int dtype, int64_t B,
                         int64_t H, int64_t N, int64_t d, int causal, double scale,
                         const int64_t *qrows, int64_t n_q, const int64_t *krows,
                         int64_t n_k, double *dq_rows, double *dk_rows,
                         double *dv_rows)
{
    const int64_t total = B * H * N;
    for (int64_t t = 0; t < n_q; ++t)
        if (qrows[t] < 0 || qrows[t] >= total) return -1;
    for (int64_t t = 0; t < n_k; ++t)
        if (krows[t] < 0 || krows[t] >= total) return -1;
    bproblem bp;
    int rc = load_bproblem(&bp, q, k, v, dO, o, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    int fail = 0;
    /* per-row D_i of every head that a sampled key belongs to */
    char *need = (char *)calloc((size_t)(B * H > 0 ? B * H : 1), 1);
    double *Dall = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    double *Lall = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    if (!need || !Dall || !Lall) {
        free(need); free(Dall); free(Lall); free_bproblem(&bp);
        return -2;
    }
    for (int64_t t = 0; t < n_k; ++t) need[krows[t] / N] = 1;
#pragma omp parallel
    {
        double *prow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *dprow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!prow || !dprow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r)
                if (need[r / N]) Dall[r] = grad_row(&bp, r / N, r % N, prow, dprow, Lall + r);
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < n_q; ++t) {
                const int64_t bh = qrows[t] / N, i = qrows[t] % N;
                const double D = grad_row(&bp, bh, i, prow, dprow, NULL);
                const int64_t nkeys = causal ? i + 1 : N;
                const double *kh = bp.p.k + bh * N * d;
                double *out = dq_rows + t * d;
                for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
                for (int64_t j = 0; j < nkeys; ++j) {
                    const double ds = prow[j] * (dprow[j] - D);
                    for (int64_t c = 0; c < d; ++c) out[c] += scale * ds * kh[j * d + c];
                }
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < n_k; ++t) {
                const int64_t bh = krows[t] / N, j = krows[t] % N;
                double *ok = dk_rows + t * d, *ov = dv_rows + t * d;
                for (int64_t c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
                const double *kj = bp.p.k + (bh * N + j) * d;
                const double *vj = bp.p.v + (bh * N + j) * d;
                for (int64_t i = causal ? j : 0; i < N; ++i) {
                    const double *qi = bp.p.q + (bh * N + i) * d;
                    const double *doi = bp.dO + (bh * N + i) * d;
                    double dot = 0.0, dp = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        dot += qi[c] * kj[c];
                        dp += doi[c] * vj[c];
                    }
                    const double pij = exp(scale * dot - Lall[bh * N + i]);
                    const double ds = pij * (dp - Dall[bh * N + i]);
                    for (int64_t c = 0; c < d; ++c) {
                        ok[c] += scale * ds * qi[c];
                        ov[c] += pij * doi[c];
                    }
                }
            }
        }
        free(prow);
        free(dprow);
    }
    free(need);
    free(Dall);
    free(Lall);
    free_bproblem(&bp);
    return fail ? -2 : 0;
}

/* ---- mask variants --------------------------------------------------------
 *
 * [P-baidu] §8 lists the mask kinds an implementation may have to support:
 * causal, padding and sliding window.  Readings (the page defines none of
 * them): query i of batch element b may attend key j when
 *     max(0, i - wl) <= j <= min(L_b - 1, i + wr),
 * where wl / wr < 0 drop that side of the window, and L_b (0..N) is the
 * element's valid length (padding: keys >= L_b are masked, and rows i >= L_b
 * have no keys at all; their output row is 0 and their lse is -inf).  Causal
 * is wl < 0, wr = 0.  seqlens (host int32 [B]) may be NULL: every L_b = N.
 */
int oracle_attn_fwd_masked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                           int64_t wl, int64_t wr, const int32_t *seqlens,
                           double scale, double *o, double *lse)
{
    if (seqlens)
        for (int64_t b = 0; b < B; ++b)
            if (seqlens[b] < 0 || seqlens[b] > N) return -1;
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, 0, scale);
    if (rc) return rc;
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / N, i = r % N, b = bh / H;
                const int64_t L = seqlens ? seqlens[b] : N;
                int64_t lo = wl < 0 ? 0 : i - wl;
                int64_t hi = wr < 0 ? L - 1 : i + wr;
                if (lo < 0) lo = 0;
                if (hi > L - 1) hi = L - 1;
                double *orow = o + r * d;
                if (i >= L || lo > hi) {
                    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                    lse[r] = -INFINITY;
                    continue;
                }
                const double *qi = p.q + r * d;
                const double *kh = p.k + bh * N * d, *vh = p.v + bh * N * d;
                double m = -INFINITY;
                for (int64_t j = lo; j <= hi; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                for (int64_t j = lo; j <= hi; ++j) {
                    const double w = exp(s[j] - m);
                    l += w;
                    for (int64_t c = 0; c < d; ++c) orow[c] += w * vh[j * d + c];
                }
                for (int64_t c = 0; c < d; ++c) orow[c] /= l;
                lse[r] = m + log(l);
            }
        }
        free(s);
    }
    free_problem(&p);
    return fail ? -2 : 0;
}

/* ---- queries against a longer run of keys (decoding) ---------------------
 *
 * "FlashAttention V2 核心原理与架构设计" (wmrh.cn) §5.1 pairs the kernel with
 * FlashDecoding for sequences beyond 32K keys, where a few new query rows
 * attend to a long cache of keys.  The page fixes no shapes; the reading
 * used here: q and o are [B,H,Nq,d], k and v are [B,H,Nk,d].  Without the
 * causal flag every query uses all Nk keys.  With it the queries are the
 * last Nq positions of the sequence, so query i may use keys
 * j <= i + (Nk - Nq) (bottom-right alignment; Nq = Nk is the square causal
 * mask).  A query with no allowed key (possible only when Nq > Nk) gets
 * o = 0 and lse = -inf. */
int oracle_attn_fwd_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                           int64_t d, int causal, double scale, double *o, double *lse)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d < 1) return -1;
    if (dtype != ORACLE_DTYPE_F16 && dtype != ORACLE_DTYPE_BF16) return -1;
    const int64_t nq = B * H * Nq * d, nk = B * H * Nk * d;
    double *qd = (double *)malloc((size_t)(nq > 0 ? nq : 1) * sizeof(double));
    double *kd = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    double *vd = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    if (!qd || !kd || !vd) {
        free(qd); free(kd); free(vd);
        return -2;
    }
    decode_all(q, dtype, nq, qd);
    decode_all(k, dtype, nk, kd);
    decode_all(v, dtype, nk, vd);
    const int64_t rows = B * H * Nq;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(Nk > 0 ? Nk : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / Nq, i = r % Nq;
                int64_t hi = causal ? i + (Nk - Nq) : Nk - 1;   /* last allowed key */
                if (hi > Nk - 1) hi = Nk - 1;
                double *orow = o + r * d;
                if (hi < 0) {
                    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                    lse[r] = -INFINITY;
                    continue;
                }
                const double *qi = qd + r * d;
                const double *kh = kd + bh * Nk * d, *vh = vd + bh * Nk * d;
                double m = -INFINITY;
                for (int64_t j = 0; j <= hi; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                for (int64_t j = 0; j <= hi; ++j) {
                    const double wj = exp(s[j] - m);
                    l += wj;
                    for (int64_t c = 0; c < d; ++c) orow[c] += wj * vh[j * d + c];
                }
                for (int64_t c = 0; c < d; ++c) orow[c] /= l;
                lse[r] = m + log(l);
            }
        }
        free(s);
    }
    free(qd); free(kd); free(vd);
    return fail ? -2 : 0;
}

/* Gradients of oracle_attn_fwd_masked for an upstream dO (same mask
 * reading): per row i with allowed keys lo..hi, P_ij = softmax of the
 * scores over those keys, dP_ij = dO_i . v_j, D_i = sum_j P_ij dP_ij (or
 * dO_i . o_i with a given 16-bit o), dS_ij = P_ij (dP_ij - D_i), and
 *     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *     dv_j = sum_i P_ij dO_i.
 * Rows without keys (i >= L_b) add nothing; keys no row may attend get 0.
 * Heads run in parallel; within a head the rows run in order. */
int oracle_attn_bwd_masked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const uint16_t *dO, const uint16_t *o, int dtype, int64_t B,
                           int64_t H, int64_t N, int64_t d, int64_t wl, int64_t wr,
                           const int32_t *seqlens, double scale, double *dq, double *dk,
                           double *dv)
{
    if (seqlens)
        for (int64_t b = 0; b < B; ++b)
            if (seqlens[b] < 0 || seqlens[b] > N) return -1;
    bproblem bp;
    int rc = load_bproblem(&bp, q, k, v, dO, o, dtype, B, H, N, d, 0, scale);
    if (rc) return rc;
    const int64_t n = B * H * N * d;
    for (int64_t t = 0; t < n; ++t) dq[t] = dk[t] = dv[t] = 0.0;
    int fail = 0;
#pragma omp parallel
    {
        double *pr = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *dpr = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!pr || !dpr) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                const int64_t L = seqlens ? seqlens[bh / H] : N;
                const double *qh = bp.p.q + bh * N * d, *kh = bp.p.k + bh * N * d;
                const double *vh = bp.p.v + bh * N * d, *doh = bp.dO + bh * N * d;
                double *dqh = dq + bh * N * d, *dkh = dk + bh * N * d, *dvh = dv + bh * N * d;
                for (int64_t i = 0; i < L; ++i) {
                    int64_t lo = wl < 0 ? 0 : i - wl;
                    int64_t hi = wr < 0 ? L - 1 : i + wr;
                    if (lo < 0) lo = 0;
                    if (hi > L - 1) hi = L - 1;
                    if (lo > hi) continue;
                    const double *qi = qh + i * d, *doi = doh + i * d;
                    double m = -INFINITY;
                    for (int64_t j = lo; j <= hi; ++j) {
                        double dot = 0.0;
                        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
                        pr[j] = scale * dot;
                        if (pr[j] > m) m = pr[j];
                    }
                    double l = 0.0;
                    for (int64_t j = lo; j <= hi; ++j) {
                        pr[j] = exp(pr[j] - m);
                        l += pr[j];
                    }
                    double D = 0.0;
                    for (int64_t j = lo; j <= hi; ++j) {
                        pr[j] /= l;
                        double dp = 0.0;
                        for (int64_t c = 0; c < d; ++c) dp += doi[c] * vh[j * d + c];
                        dpr[j] = dp;
                        D += pr[j] * dp;
                    }
                    if (bp.o) {
                        const double *oi = bp.o + (bh * N + i) * d;
                        D = 0.0;
                        for (int64_t c = 0; c < d; ++c) D += doi[c] * oi[c];
                    }
                    for (int64_t j = lo; j <= hi; ++j) {
                        const double ds = pr[j] * (dpr[j] - D);
                        for (int64_t c = 0; c < d; ++c) {
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qi[c];
                            dvh[j * d + c] += pr[j] * doi[c];
                        }
                    }
                }
            }
        }
        free(pr);
        free(dpr);
    }
    free_bproblem(&bp);
    return fail ? -2 : 0;
}

/* ---- dropout ---------------------------------------------------------------
 *
 * The pages list dropout among the operations fused into the attention
 * kernel and warn that forward and backward must draw the same random
 * pattern ([P-wmrh] §1.2 kernel fusion, §4.2 problem 3).  Readings (the pages
 * fix no generator or mapping): the generator is Philox4x32-10 (Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC 2011), written here from that definition:
 *   per round, with M0 = 0xD2511F53, M1 = 0xCD9E8D57,
 *     (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2   (64-bit products)
 *     c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
 *   and before every round but the first the key gains
 *     (k0, k1) += (0x9E3779B9, 0xBB67AE85)   (mod 2^32).
 * Element (b, h, i, j) of the weights P is kept when its byte is below
 * T = round((1 - p) * 256), where the 16 bytes of one call with
 *   counter = (i, 2 * (j / 32) + ((j / 4) % 2), b * H + h, offset),
 *   key     = (seed low 32 bits, seed high 32 bits)
 * are, little-endian in the output words, the keys
 *   j' = 32 * (j / 32) + 8 * g + 4 * ((j / 4) % 2) + e  at byte 4 g + e.
 * Kept weights are scaled by 256 / T, so E[kept weight] is the weight; the
 * row sum l and lse stay those of the undropped weights (dropout acts after
 * the softmax).  T = 0 drops everything (o = 0).
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The byte that decides element (bh, i, j). */
static unsigned dropout_byte(int64_t bh, int64_t i, int64_t j, uint64_t seed,
                             uint32_t offset)
{
    const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(2 * (j / 32) + (j / 4) % 2),
                             (uint32_t)bh, offset};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const int64_t jj = j % 32;
    const int g = (int)(jj / 8), e = (int)(jj % 4);
    return (out[g] >> (8 * e)) & 0xffu;
}

/* Keep factor Z_ij: 256 / T if kept, else 0 (T = round((1 - p) 256)). */
static double dropout_factor(int64_t bh, int64_t i, int64_t j, uint64_t seed,
                             uint32_t offset, int T)
{
    if (T <= 0) return 0.0;
    return dropout_byte(bh, i, j, seed, offset) < (unsigned)T ? 256.0 / T : 0.0;
}

/* The keep factors Z of one head-row range, for tests: z[(bh*N + i)*N + j]. */
int oracle_dropout_factors(int64_t BH, int64_t N, uint64_t seed, uint32_t offset, int T,
                           double *z)
{
    if (T < 0 || T > 256) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < BH * N; ++r)
        for (int64_t j = 0; j < N; ++j)
            z[r * N + j] = dropout_factor(r / N, r % N, j, seed, offset, T);
    return 0;
}

/* Flat row r = (b*H+h)*N + i with dropout: o_i = sum_j P_ij Z_ij v_j into
 * orow, lse as without dropout into *lse; s is scratch for N scores. */
static void dropout_fwd_row(const problem *p, int64_t r, double *s, int T, uint64_t seed,
                            uint32_t offset, double *orow, double *lse)
{
    const int64_t N = p->N, d = p->d;
    const int64_t bh = r / N, i = r % N;
    const double *qi = p->q + r * d;
    const double *kh = p->k + bh * N * d, *vh = p->v + bh * N * d;
    const int64_t nkeys = p->causal ? i + 1 : N;
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
        s[j] = p->scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) l += exp(s[j] - m);
    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double w = exp(s[j] - m) / l * dropout_factor(bh, i, j, seed, offset, T);
        if (w == 0.0) continue;
        for (int64_t c = 0; c < d; ++c) orow[c] += w * vh[j * d + c];
    }
    *lse = m + log(l);
}

/* Forward with dropout: o_i = sum_j P_ij Z_ij v_j, lse as without dropout. */
int oracle_attn_fwd_dropout(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                            int causal, double scale, int T, uint64_t seed,
                            uint32_t offset, double *o, double *lse)
{
    if (T < 0 || T > 256) return -1;
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r)
                dropout_fwd_row(&p, r, s, T, seed, offset, o + r * d, lse + r);
        }
        free(s);
    }
    free_problem(&p);
    return fail ? -2 : 0;
}

/* The same on the flat rows rows[] only: o_rows [n_rows, d], lse_rows. */
int oracle_attn_fwd_dropout_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                                 int causal, double scale, int T, uint64_t seed,
                                 uint32_t offset, const int64_t *rows, int64_t n_rows,
                                 double *o_rows, double *lse_rows)
{
    if (T < 0 || T > 256) return -1;
    for (int64_t t = 0; t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * N) return -1;
    problem p;
    int rc = load_problem(&p, q, k, v, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < n_rows; ++t)
                dropout_fwd_row(&p, rows[t], s, T, seed, offset, o_rows + t * d, lse_rows + t);
        }
        free(s);
    }
    free_problem(&p);
    return fail ? -2 : 0;
}

/* Backward with dropout, the row term from a given 16-bit o (as the kernel
 * is handed the forward's output):
 *   dV_j = sum_i P_ij Z_ij dO_i,  dP_ij = dO_i . v_j,
 *   dS_ij = P_ij (Z_ij dP_ij - D_i),  D_i = dO_i . o_i
 *   (= sum_j P_ij Z_ij dP_ij for the exact o), dQ, dK as without dropout. */
int oracle_attn_bwd_dropout(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const uint16_t *dO, const uint16_t *o, int dtype, int64_t B,
                            int64_t H, int64_t N, int64_t d, int causal, double scale,
                            int T, uint64_t seed, uint32_t offset, double *dq, double *dk,
                            double *dv)
{
    if (T < 0 || T > 256 || !o) return -1;
    bproblem bp;
    int rc = load_bproblem(&bp, q, k, v, dO, o, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    const int64_t n = B * H * N * d;
    for (int64_t t = 0; t < n; ++t) dq[t] = dk[t] = dv[t] = 0.0;
    int fail = 0;
#pragma omp parallel
    {
        double *prow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *dprow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!prow || !dprow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                const double *qh = bp.p.q + bh * N * d, *kh = bp.p.k + bh * N * d;
                const double *doh = bp.dO + bh * N * d;
                double *dqh = dq + bh * N * d, *dkh = dk + bh * N * d, *dvh = dv + bh * N * d;
                for (int64_t i = 0; i < N; ++i) {
                    /* P_i. and dP_i.; with o given, grad_row returns dO_i . o_i */
                    const double D = grad_row(&bp, bh, i, prow, dprow, NULL);
                    const int64_t nkeys = causal ? i + 1 : N;
                    for (int64_t j = 0; j < nkeys; ++j) {
                        const double z = dropout_factor(bh, i, j, seed, offset, T);
                        const double ds = prow[j] * (z * dprow[j] - D);
                        for (int64_t c = 0; c < d; ++c) {
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qh[i * d + c];
                            dvh[j * d + c] += prow[j] * z * doh[i * d + c];
                        }
                    }
                }
            }
        }
        free(prow);
        free(dprow);
    }
    free_bproblem(&bp);
    return fail ? -2 : 0;
}

/* Sampled dropout gradients (o given, as oracle_attn_bwd_dropout): dq for
 * the flat query rows qrows[], dk and dv for the flat key rows krows[],
 * packed [n_q,d] and [n_k,d].  As in oracle_attn_bwd_rows, the heads of the
 * sampled keys are evaluated row by row first (lse_i and D_i kept). */
int oracle_attn_bwd_dropout_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *dO, const uint16_t *o, int dtype, int64_t B,
                                 int64_t H, int64_t N, int64_t d, int causal, double scale,
                                 int T, uint64_t seed, uint32_t offset, const int64_t *qrows,
                                 int64_t n_q, const int64_t *krows, int64_t n_k,
                                 double *dq_rows, double *dk_rows, double *dv_rows)
{
    if (T < 0 || T > 256 || !o) return -1;
    const int64_t total = B * H * N;
    for (int64_t t = 0; t < n_q; ++t)
        if (qrows[t] < 0 || qrows[t] >= total) return -1;
    for (int64_t t = 0; t < n_k; ++t)
        if (krows[t] < 0 || krows[t] >= total) return -1;
    bproblem bp;
    int rc = load_bproblem(&bp, q, k, v, dO, o, dtype, B, H, N, d, causal, scale);
    if (rc) return rc;
    int fail = 0;
    char *need = (char *)calloc((size_t)(B * H > 0 ? B * H : 1), 1);
    double *Dall = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    double *Lall = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    if (!need || !Dall || !Lall) {
        free(need); free(Dall); free(Lall); free_bproblem(&bp);
        return -2;
    }
    for (int64_t t = 0; t < n_k; ++t) need[krows[t] / N] = 1;
#pragma omp parallel
    {
        double *prow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *dprow = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!prow || !dprow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r)
                if (need[r / N]) Dall[r] = grad_row(&bp, r / N, r % N, prow, dprow, Lall + r);
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < n_q; ++t) {
                const int64_t bh = qrows[t] / N, i = qrows[t] % N;
                const double D = grad_row(&bp, bh, i, prow, dprow, NULL);
                const int64_t nkeys = causal ? i + 1 : N;
                const double *kh = bp.p.k + bh * N * d;
                double *out = dq_rows + t * d;
                for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
                for (int64_t j = 0; j < nkeys; ++j) {
                    const double z = dropout_factor(bh, i, j, seed, offset, T);
                    const double ds = prow[j] * (z * dprow[j] - D);
                    for (int64_t c = 0; c < d; ++c) out[c] += scale * ds * kh[j * d + c];
                }
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < n_k; ++t) {
                const int64_t bh = krows[t] / N, j = krows[t] % N;
                double *ok = dk_rows + t * d, *ov = dv_rows + t * d;
                for (int64_t c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
                const double *kj = bp.p.k + (bh * N + j) * d;
                const double *vj = bp.p.v + (bh * N + j) * d;
                for (int64_t i = causal ? j : 0; i < N; ++i) {
                    const double *qi = bp.p.q + (bh * N + i) * d;
                    const double *doi = bp.dO + (bh * N + i) * d;
                    double dot = 0.0, dp = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        dot += qi[c] * kj[c];
                        dp += doi[c] * vj[c];
                    }
                    const double pij = exp(scale * dot - Lall[bh * N + i]);
                    const double z = dropout_factor(bh, i, j, seed, offset, T);
                    const double ds = pij * (z * dp - Dall[bh * N + i]);
                    for (int64_t c = 0; c < d; ++c) {
                        ok[c] += scale * ds * qi[c];
                        ov[c] += pij * z * doi[c];
                    }
                }
            }
        }
        free(prow);
        free(dprow);
    }
    free(need);
    free(Dall);
    free(Lall);
    free_bproblem(&bp);
    return fail ? -2 : 0;
}
