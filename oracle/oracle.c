/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY. Not part of the product path.
 *
 * A plain, slow, obviously correct fp64 CPU implementation of what the
 * block-dequant GEMV computes. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call it. It shares no code, header,
 * table or constant with the HIP library: it reads the canonical GGUF-style
 * block bytes directly and writes everything out by the definitions.
 *
 * What is computed (the plain definition that the fused kernels reorder):
 *   W[n][k] = d(n, k/32) * v(n, k)         dequantised weight, exact in double
 *   y[n]    = sum_{k<K} W[n][k] * x[k]      natural k order, in double
 *   a[n]    = sum_{k<K} |W[n][k] * x[k]|    magnitude sum used by the tolerance
 *
 * Sources (pages, not code):
 *  - "EdgeRunner beats llama.cpp" (chriskarani.xyz), section "What worked",
 *    item 2 "Fused Q8_0 dequant + GEMV": weights are read quantised and the
 *    dequantisation happens inside the matrix-vector product, with no float
 *    copy of the weights. The oracle is the unfused definition of that product.
 *  - RunIT_Mac README, optimisation table: Q8_0 costs 1.06 bytes per weight and
 *    Q4_0 0.56, i.e. 34 B and 18 B per 32-weight block (one fp16 scale each).
 *  - RunIT_Mac README, kernel table: the GEMVs take fp32 activations and write
 *    fp32 outputs ("f32in_f32out"); the data-flow figure accumulates in f32.
 *  - robotnurse.io "We wrote our own inference engine", "Correctness first":
 *    a slow reference of every layer is kept beside the GPU kernels as a
 *    parity gate. This file is that reference for the GEMV.
 *  - RunIT_Mac README, "Fused gate+up+silu": the gate and up projections and
 *    the SiLU product are one step; out = silu(gate) * up.
 *  - RunIT_Mac README, optimisation table and data-flow figure: the fused QKV
 *    projection adds its bias in the same dispatch ("Fused QKV+bias"), and the
 *    model keeps an f32 residual stream that projections add into;
 *    robotnurse.io "We wrote our own inference engine", "What actually moved
 *    it", item 5: some GEMVs write fp16 outputs. oracle_gemv_epilogue is the
 *    product followed by those additions, in double.
 *  - RunIT_Mac README, kernel table ("Fused Q4_K dequant + GEMV") and
 *    quantisation table (Q4_K_M), EdgeRunner "Run it yourself" (loads Q4_K_M):
 *    the Q4_K super-block, whose layout the pages do not give; it is read as
 *    the published GGUF k-quant block (q4_k_weight below).
 *  - RunIT_Mac README, quantisation table (Q6_K supported) and the data-flow
 *    note on Q8_0/Q5K/Q6K weights, EdgeRunner "Run it yourself" (loads Q6_K):
 *    the Q6_K super-block, likewise not described on the pages and read as the
 *    published GGUF block (q6_k_weight below).
 *  - RunIT_Mac README, kernel table and data-flow figure: RMSNorm with f32
 *    input, output and gamma precedes the projections; "EdgeRunner beats
 *    llama.cpp", The progression, fused it into the GEMV (RMSNorm+GEMV).
 *    oracle_rmsnorm and oracle_gemv_rmsnorm write that out in double.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - Block field order is the GGUF one: little-endian fp16 scale first, then
 *    the quants.  Q8_0 quants are int8, the full range -128..127 is accepted.
 *  - Q4_0: byte j (0..15) of the quant field holds element j in its low nibble
 *    and element j+16 in its high nibble (GGUF convention); value = nibble - 8.
 *  - fp16 decoding follows IEEE 754 binary16 exactly, subnormals included.
 *  - silu(g) = g / (1 + exp(-g)).
 *  - RMSNorm: out[k] = gamma[k] * x[k] / sqrt(mean(x^2) + eps), with eps >= 0
 *    given by the caller (the pages name the operation, not its epsilon).
 *
 * Exactness: the fp16 decode, the int->double conversion, d*q (<= 19
 * significant bits) and (d*q)*x (<= 43 bits) are all exact in double, so the
 * only rounding is in the running sum: |y - exact| <= K * 2^-53 * a[n].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_Q8_0 = 1, ORACLE_Q4_0 = 2, ORACLE_F16 = 3, ORACLE_Q4_K = 4, ORACLE_Q6_K = 5 };

/* IEEE 754 binary16 -> double, exact. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero and subnormals */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static uint16_t read_le16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Dequantised weight of element i (0..31) of one canonical block. */
static double q8_0_weight(const uint8_t *blk, int i)
{
    double d = oracle_half_to_double(read_le16(blk));
    int q = (int)(int8_t)blk[2 + i];
    return d * (double)q;
}

static double q4_0_weight(const uint8_t *blk, int i)
{
    double d = oracle_half_to_double(read_le16(blk));
    const uint8_t *qs = blk + 2;
    int nib = (i < 16) ? (qs[i] & 0x0f) : (qs[i - 16] >> 4);
    return d * (double)(nib - 8);
}

/* Q4_K super-block (256 weights, 144 bytes; the GGUF k-quant block the pages
 * name as Q4_K / Q4_K_M without describing it, read here as published for
 * GGUF): fp16 d, fp16 dmin, 12 bytes holding eight 6-bit scales sc[j] and
 * eight 6-bit mins mn[j] (one pair per sub-block of 32 weights), then 128
 * bytes of 4-bit quants. Weight i of sub-block j = i / 32:
 *   w = d * sc[j] * q_i - dmin * mn[j]
 * Scale/min bytes u[0..11]: for j < 4, sc[j] = low 6 bits of u[j] and mn[j] =
 * low 6 bits of u[j + 4]; for j >= 4, sc[j] = low nibble of u[j + 4] plus the
 * top two bits of u[j - 4] as bits 4-5, and mn[j] = high nibble of u[j + 4]
 * plus the top two bits of u[j] as bits 4-5. Quants: weights 64g .. 64g + 63
 * use bytes 32g .. 32g + 31, weight 64g + l in the low nibble of byte 32g + l
 * and weight 64g + 32 + l in its high nibble. d * sc * q (<= 21 significant
 * bits) and dmin * mn (<= 17) are exact in double, and so is their
 * difference, so w is exact. */
static void q4_k_scale_min(const uint8_t *u, int j, int *sc, int *mn)
{
    if (j < 4) {
        *sc = u[j] & 63;
        *mn = u[j + 4] & 63;
    } else {
        *sc = (u[j + 4] & 15) | ((u[j - 4] >> 6) << 4);
        *mn = (u[j + 4] >> 4) | ((u[j] >> 6) << 4);
    }
}

static double q4_k_weight(const uint8_t *blk, int i)
{
    double d = oracle_half_to_double(read_le16(blk));
    double dmin = oracle_half_to_double(read_le16(blk + 2));
    int sc, mn;
    q4_k_scale_min(blk + 4, i / 32, &sc, &mn);
    const uint8_t *qs = blk + 16;
    int g = i / 64, l = i % 64;
    int q = (l < 32) ? (qs[32 * g + l] & 15) : (qs[32 * g + l - 32] >> 4);
    return d * (double)sc * (double)q - dmin * (double)mn;
}

/* Q6_K super-block (256 weights, 210 bytes; the GGUF k-quant block the pages
 * name as Q6_K without describing it, read here as published for GGUF): 128
 * bytes ql of low 4-bit parts, 64 bytes qh of high 2-bit parts, sixteen int8
 * scales sc[0..15] (one per 16 weights), then the fp16 d. Weight i lies in
 * half h = i / 128; with r = i % 128, group g = r / 32 and l = r % 32 its low 4
 * bits are the low (g < 2) or high (g >= 2) nibble of ql[64h + 32(g % 2) + l]
 * and its high 2 bits are bits 2g, 2g + 1 of qh[32h + l]:
 *   q = low | high << 4 (0..63),   w = d * sc[i / 16] * (q - 32)
 * d * sc * (q - 32) has <= 25 significant bits: exact in double. */
static double q6_k_weight(const uint8_t *blk, int i)
{
    const uint8_t *ql = blk, *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    double d = oracle_half_to_double(read_le16(blk + 208));
    int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
    int lo = ql[64 * h + 32 * (g % 2) + l];
    lo = (g < 2) ? (lo & 15) : (lo >> 4);
    int hi = (qh[32 * h + l] >> (2 * g)) & 3;
    int q = lo | (hi << 4);
    return d * (double)sc[i / 16] * (double)(q - 32);
}

/* W[n][k] of an N x K matrix of `kind` from its canonical bytes w (rows of
 * K/32 blocks, K/256 super-blocks or K fp16 values). */
static double weight_at(int kind, const uint8_t *w, int64_t n, int64_t k, int64_t K)
{
    if (kind == ORACLE_Q8_0)
        return q8_0_weight(w + (n * (K / 32) + k / 32) * 34, (int)(k % 32));
    if (kind == ORACLE_Q4_0)
        return q4_0_weight(w + (n * (K / 32) + k / 32) * 18, (int)(k % 32));
    if (kind == ORACLE_Q4_K)
        return q4_k_weight(w + (n * (K / 256) + k / 256) * 144, (int)(k % 256));
    if (kind == ORACLE_Q6_K)
        return q6_k_weight(w + (n * (K / 256) + k / 256) * 210, (int)(k % 256));
    return oracle_half_to_double(read_le16(w + (n * K + k) * 2));
}

/* One output row: y = sum W[n][k] x[k], a = sum |W[n][k] x[k]|. */
static void one_row(int kind, const uint8_t *w, const float *x, int64_t n, int64_t K,
                    double *y, double *a)
{
    double sum = 0.0, asum = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double wk = weight_at(kind, w, n, k, K);
        double p = wk * (double)x[k];
        sum += p;
        asum += fabs(p);
    }
    *y = sum;
    *a = asum;
}

static int bad_args(int kind, int64_t N, int64_t K)
{
    if (N < 0 || K < 0) return 1;
    if (kind != ORACLE_Q8_0 && kind != ORACLE_Q4_0 && kind != ORACLE_F16 && kind != ORACLE_Q4_K &&
        kind != ORACLE_Q6_K)
        return 1;
    if (kind != ORACLE_F16 && K % 32 != 0) return 1;
    if ((kind == ORACLE_Q4_K || kind == ORACLE_Q6_K) && K % 256 != 0) return 1;
    return 0;
}

/* Rows [r0, r1) of y = W x. */
int oracle_gemv_range(int kind, const void *w, const float *x, double *y, double *a,
                      int64_t N, int64_t K, int64_t r0, int64_t r1)
{
    if (bad_args(kind, N, K) || r0 < 0 || r1 > N || r0 > r1) return 1;
    for (int64_t n = r0; n < r1; ++n)
        one_row(kind, (const uint8_t *)w, x, n, K, &y[n], a ? &a[n] : &(double){0});
    return 0;
}

/* A chosen list of rows: y[i], a[i] belong to row rows[i]. */
int oracle_gemv_rows(int kind, const void *w, const float *x, const int64_t *rows,
                     int64_t nrows, double *y, double *a, int64_t N, int64_t K)
{
    if (bad_args(kind, N, K)) return 1;
    for (int64_t i = 0; i < nrows; ++i) {
        if (rows[i] < 0 || rows[i] >= N) return 1;
        double dummy;
        one_row(kind, (const uint8_t *)w, x, rows[i], K, &y[i], a ? &a[i] : &dummy);
    }
    return 0;
}

/* ---- static row ranges over plain pthreads ------------------------------ */

struct job {
    int kind;
    const void *w;
    const float *x;
    double *y, *a;
    int64_t N, K, r0, r1;
};

static void *job_main(void *p)
{
    struct job *j = (struct job *)p;
    oracle_gemv_range(j->kind, j->w, j->x, j->y, j->a, j->N, j->K, j->r0, j->r1);
    return NULL;
}

/* y = W x over all N rows, split into nthreads equal static row ranges. */
int oracle_gemv(int kind, const void *w, const float *x, double *y, double *a,
                int64_t N, int64_t K, int nthreads)
{
    if (bad_args(kind, N, K)) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || N < nthreads)
        return oracle_gemv_range(kind, w, x, y, a, N, K, 0, N);
    pthread_t tid[256];
    struct job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct job){kind, w, x, y, a, N, K, N * t / nthreads, N * (t + 1) / nthreads};
        if (pthread_create(&tid[t], NULL, job_main, &jobs[t]) != 0) {
            job_main(&jobs[t]);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t]) pthread_join(tid[t], NULL);
    return 0;
}

/* ---- gate/up with the SiLU product -------------------------------------- */

double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/* out[n] = silu(g[n]) * u[n], g = Wgate x, u = Wup x. g, u, ag, au may be
 * returned for tolerance propagation (pass NULL to skip). */
int oracle_gateup_silu(int kind, const void *gate, const void *up, const float *x,
                       double *out, double *g, double *u, double *ag, double *au,
                       int64_t N_ff, int64_t K, int nthreads)
{
    if (kind == ORACLE_F16 || bad_args(kind, N_ff, K)) return 1;
    double *gg = g ? g : (double *)malloc(sizeof(double) * (size_t)(N_ff ? N_ff : 1));
    double *uu = u ? u : (double *)malloc(sizeof(double) * (size_t)(N_ff ? N_ff : 1));
    double *aag = ag ? ag : (double *)malloc(sizeof(double) * (size_t)(N_ff ? N_ff : 1));
    double *aau = au ? au : (double *)malloc(sizeof(double) * (size_t)(N_ff ? N_ff : 1));
    int rc = 1;
    if (gg && uu && aag && aau) {
        rc = oracle_gemv(kind, gate, x, gg, aag, N_ff, K, nthreads);
        if (!rc) rc = oracle_gemv(kind, up, x, uu, aau, N_ff, K, nthreads);
        if (!rc)
            for (int64_t n = 0; n < N_ff; ++n) out[n] = oracle_silu(gg[n]) * uu[n];
    }
    if (!g) free(gg);
    if (!u) free(uu);
    if (!ag) free(aag);
    if (!au) free(aau);
    return rc;
}

/* ---- multi-row "verify": each activation row on its own ----------------- */

/* Y[m][n] = sum_k W[n][k] X[m][k] for m < M; row m is exactly the M=1 result
 * for X[m], which is what the verify pass must reproduce. */
int oracle_verify(int kind, const void *w, const float *X, double *Y, double *A,
                  int64_t N, int64_t K, int M, int nthreads)
{
    if (M < 1 || bad_args(kind, N, K)) return 1;
    for (int m = 0; m < M; ++m) {
        int rc = oracle_gemv(kind, w, X + (int64_t)m * K, Y + (int64_t)m * N,
                             A ? A + (int64_t)m * N : NULL, N, K, nthreads);
        if (rc) return rc;
    }
    return 0;
}

/* Epilogue variants of the product: out[n] = y[n] + bias[n] + residual[n], in
 * double, with either addend absent when its pointer is NULL. An fp16 output
 * is not rounded here: the oracle keeps the exact value and the tests bound
 * the fp16 rounding on top of the linear tolerance. a[n] is the product's
 * magnitude sum, as for oracle_gemv. */
int oracle_gemv_epilogue(int kind, const void *w, const float *x, const float *bias, const float *residual,
                         double *out, double *a, int64_t N, int64_t K, int threads)
{
    int rc = oracle_gemv(kind, w, x, out, a, N, K, threads);
    if (rc)
        return rc;
    for (int64_t n = 0; n < N; ++n) {
        if (bias)
            out[n] += (double)bias[n];
        if (residual)
            out[n] += (double)residual[n];
    }
    return 0;
}

/* ---- RMSNorm and the RMSNorm-prologue product ---------------------------- */

/* RMSNorm of one activation vector, in double (RunIT_Mac README, kernel table
 * and data-flow figure: RMSNorm takes an f32 input and an f32 gamma and gives
 * an f32 output; "EdgeRunner beats llama.cpp", The progression: the RMSNorm
 * that precedes a projection fused into that GEMV):
 *   out[k] = gamma[k] * x[k] / sqrt((1/K) * sum_j x[j]^2 + eps)
 * eps >= 0 is the caller's (the pages give no value). */
int oracle_rmsnorm(const float *x, const float *gamma, double eps, double *out, int64_t K)
{
    if (K <= 0 || !(eps >= 0.0))
        return 1;
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k)
        ss += (double)x[k] * (double)x[k];
    double rms = sqrt(ss / (double)K + eps);
    for (int64_t k = 0; k < K; ++k)
        out[k] = (double)gamma[k] * (double)x[k] / rms;
    return 0;
}

/* y = W * rmsnorm(x): the product of the normalised activation (kept exact in
 * double) with the dequantised weights, plus a[n] = sum_k |W[n][k] * xn[k]|. */
int oracle_gemv_rmsnorm(int kind, const void *w, const float *x, const float *gamma, double eps,
                        double *y, double *a, int64_t N, int64_t K)
{
    if (bad_args(kind, N, K) || K == 0)
        return 1;
    double *xn = (double *)malloc(sizeof(double) * (size_t)K);
    if (!xn)
        return 1;
    int rc = oracle_rmsnorm(x, gamma, eps, xn, K);
    const uint8_t *wb = (const uint8_t *)w;
    for (int64_t n = 0; !rc && n < N; ++n) {
        double sum = 0.0, asum = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double wk = weight_at(kind, wb, n, k, K);
            double p = wk * xn[k];
            sum += p;
            asum += fabs(p);
        }
        y[n] = sum;
        if (a)
            a[n] = asum;
    }
    free(xn);
    return rc;
}

/* The gate|up SiLU product on the normalised activation: out[n] =
 * silu(g[n]) * u[n] with g = Wgate * rmsnorm(x), u = Wup * rmsnorm(x). */
int oracle_gateup_silu_rmsnorm(int kind, const void *gate, const void *up, const float *x, const float *gamma,
                               double eps, double *out, double *g, double *u, double *ag, double *au,
                               int64_t N_ff, int64_t K)
{
    if (kind == ORACLE_F16)
        return 1;
    int rc = oracle_gemv_rmsnorm(kind, gate, x, gamma, eps, g, ag, N_ff, K);
    if (!rc)
        rc = oracle_gemv_rmsnorm(kind, up, x, gamma, eps, u, au, N_ff, K);
    for (int64_t n = 0; !rc && n < N_ff; ++n)
        out[n] = oracle_silu(g[n]) * u[n];
    return rc;
}
