/*
 * oracle.c -- fp64 CPU oracle for the batch-invariant GEMM and for the
 * decode attention that the same pages pair with it (at the end of the file).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes is the plain definition of the GEMM as the article
 * "DeepSeek V4的batch invariance：大模型确定性推理的工程基石" states it in
 * section 2.1: C[i][j] = sum over k of A[i][k] * B[k][j], with alpha = 1 and
 * beta = 0 (the wmrh.cn V4 engineering blog, section 3.1).  Every input code
 * is first decoded to the exact real number it encodes, every product and
 * every partial sum is formed in IEEE binary64, and the sum runs over k in
 * ascending order.  Alongside C it returns S = sum_k |a_k * b_k|, the scale
 * of the error bound, and a direct binary64 -> bf16 round-to-nearest-even
 * (no detour through binary32, so no double rounding).
 *
 * Decoders follow the published format definitions:
 *   bf16     : the upper 16 bits of an IEEE binary32.
 *   e4m3fn   : OCP 8-bit float, 1 sign, 4 exponent (bias 7), 3 mantissa,
 *              subnormals m * 2^-9, no infinities, S.1111.111 is NaN.
 *   e2m1     : OCP 4-bit float, 1 sign, 2 exponent (bias 1), 1 mantissa,
 *              values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *
 * Parallelism: OpenMP over independent (row, column-chunk) tasks; inside a
 * task each output element is still a single sequential k-ascending sum, so
 * threading does not change any result.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_NCHUNK 256

/* ---------------------------------------------------------------- decoders */

double ora_dec_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double ora_dec_e4m3fn(uint8_t q)
{
    int s = (q >> 7) & 1;
    int e = (q >> 3) & 15;
    int m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

double ora_dec_e2m1(uint8_t nib)
{
    int s = (nib >> 3) & 1;
    int e = (nib >> 1) & 3;
    int m = nib & 1;
    double v;
    if (e == 0)
        v = 0.5 * m;                           /* m/2 * 2^(1-1) */
    else
        v = ldexp(1.0 + m / 2.0, e - 1);
    return s ? -v : v;
}

/* binary64 -> bf16, round to nearest, ties to even, done in one step.
 * A value x with |x| in [2^e, 2^(e+1)) has bf16 quantum 2^(e-7) (8
 * significant bits); below 2^-126 the quantum stays 2^-133 (subnormals).
 * q = |x| / quantum is computed exactly (power-of-two scaling) and rounded
 * once with nearbyint() in the default round-to-nearest-even mode. */
uint16_t ora_rne_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e2;
    frexp(a, &e2);                              /* a in [2^(e2-1), 2^e2) */
    int ue = e2 - 1;
    if (ue < -126)
        ue = -126;
    double q = nearbyint(ldexp(a, 7 - ue));     /* integer, 0..256 */
    int64_t iq = (int64_t)q;
    int64_t bits;
    if (ue == -126)
        bits = iq;                              /* exponent field 0 or 1 */
    else
        bits = ((int64_t)(ue + 127) << 7) + (iq - 128);
    if (bits >= 0x7F80)
        bits = 0x7F80;                          /* overflow -> infinity */
    return (uint16_t)(sign | (uint16_t)bits);
}

void ora_round_bf16(int64_t n, const double* x, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_rne_bf16(x[i]);
}

int ora_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the parallel loops below (host timing only: every output
 * element is computed by one thread in the same order whatever the count). */
void ora_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ GEMMs
 * Output C and S are M x N row-major with row stride ldc (elements).
 * Each task owns row m and columns [n0, n1); it sweeps k = 0..K-1 in
 * ascending order and keeps one fp64 running sum per output element.
 */

void ora_gemm_bf16(int64_t M, int64_t N, int64_t K,
                   const uint16_t* A, int64_t lda,
                   const uint16_t* B, int64_t ldb,
                   double* C, double* S, int64_t ldc)
{
    int64_t nchunks = (N + ORA_NCHUNK - 1) / ORA_NCHUNK;
    int64_t ntask = M * nchunks;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
        int64_t m = t / nchunks;
        int64_t n0 = (t % nchunks) * ORA_NCHUNK;
        int64_t n1 = n0 + ORA_NCHUNK < N ? n0 + ORA_NCHUNK : N;
        double* c = C + m * ldc;
        double* s = S + m * ldc;
        for (int64_t n = n0; n < n1; ++n) {
            c[n] = 0.0;
            s[n] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            double a = ora_dec_bf16(A[m * lda + k]);
            const uint16_t* brow = B + k * ldb;
            for (int64_t n = n0; n < n1; ++n) {
                double p = a * ora_dec_bf16(brow[n]);
                c[n] += p;
                s[n] += fabs(p);
            }
        }
    }
}

/* fp8 e4m3fn with block scales: a = dec(qA[m,k]) * sA[m, k/128],
 * b = dec(qB[k,n]) * sB[k/128, n/128]. */
void ora_gemm_fp8bs(int64_t M, int64_t N, int64_t K,
                    const uint8_t* A, int64_t lda, const float* sA, int64_t ldsa,
                    const uint8_t* B, int64_t ldb, const float* sB, int64_t ldsb,
                    double* C, double* S, int64_t ldc)
{
    int64_t nchunks = (N + ORA_NCHUNK - 1) / ORA_NCHUNK;
    int64_t ntask = M * nchunks;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
        int64_t m = t / nchunks;
        int64_t n0 = (t % nchunks) * ORA_NCHUNK;
        int64_t n1 = n0 + ORA_NCHUNK < N ? n0 + ORA_NCHUNK : N;
        double* c = C + m * ldc;
        double* s = S + m * ldc;
        for (int64_t n = n0; n < n1; ++n) {
            c[n] = 0.0;
            s[n] = 0.0;
        }
        double e4m3[256];                      /* ora_dec_e4m3fn of every code */
        for (int q = 0; q < 256; ++q)
            e4m3[q] = ora_dec_e4m3fn((uint8_t)q);
        for (int64_t k = 0; k < K; ++k) {
            double a = e4m3[A[m * lda + k]] * (double)sA[m * ldsa + k / 128];
            const uint8_t* brow = B + k * ldb;
            const float* srow = sB + (k / 128) * ldsb;
            for (int64_t n = n0; n < n1; ++n) {
                double b = e4m3[brow[n]] * (double)srow[n / 128];
                double p = a * b;
                c[n] += p;
                s[n] += fabs(p);
            }
        }
    }
}

/* E8M0 (OCP MX shared scale): 2^(e - 127); e = 255 is NaN. */
double ora_dec_e8m0(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* W4A8: a = dec_e4m3fn(qA[m,k]) * sA[m, k/128];
 *       b = dec_e2m1(code(k,n)) * dec_e8m0(sE[k/32, n])   (OCP MXFP4 weights). */
void ora_gemm_w4a8(int64_t M, int64_t N, int64_t K,
                   const uint8_t* qA, int64_t lda, const float* sA, int64_t ldsa,
                   const uint8_t* Bq, int64_t ldbq, const uint8_t* sE, int64_t ldse,
                   double* C, double* S, int64_t ldc)
{
    int64_t nchunks = (N + ORA_NCHUNK - 1) / ORA_NCHUNK;
    int64_t ntask = M * nchunks;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
        int64_t m = t / nchunks;
        int64_t n0 = (t % nchunks) * ORA_NCHUNK;
        int64_t n1 = n0 + ORA_NCHUNK < N ? n0 + ORA_NCHUNK : N;
        double* c = C + m * ldc;
        double* s = S + m * ldc;
        for (int64_t n = n0; n < n1; ++n) {
            c[n] = 0.0;
            s[n] = 0.0;
        }
        double e4m3[256], e8m0[256], e2m1[16]; /* the decoders' values of every code */
        for (int q = 0; q < 256; ++q) {
            e4m3[q] = ora_dec_e4m3fn((uint8_t)q);
            e8m0[q] = ora_dec_e8m0((uint8_t)q);
        }
        for (int q = 0; q < 16; ++q)
            e2m1[q] = ora_dec_e2m1((uint8_t)q);
        for (int64_t k = 0; k < K; ++k) {
            double a = e4m3[qA[m * lda + k]] * (double)sA[m * ldsa + k / 128];
            const uint8_t* brow = Bq + k * ldbq;
            const uint8_t* srow = sE + (k / 32) * ldse;
            for (int64_t n = n0; n < n1; ++n) {
                uint8_t code = (uint8_t)((brow[n / 2] >> (4 * (n & 1))) & 15);
                double b = e2m1[code] * e8m0[srow[n]];
                double p = a * b;
                c[n] += p;
                s[n] += fabs(p);
            }
        }
    }
}

/* fp4 weight-only: a = dec_bf16(A[m,k]); b = dec_e2m1(code(k,n)) * dec_e4m3fn(sB[k/32, n]).
 * code(k,n) is the low nibble of byte Bq[k, n/2] for even n, the high nibble for odd n. */
void ora_gemm_fp4w(int64_t M, int64_t N, int64_t K,
                   const uint16_t* A, int64_t lda,
                   const uint8_t* Bq, int64_t ldbq, const uint8_t* sB, int64_t ldsb,
                   double* C, double* S, int64_t ldc)
{
    int64_t nchunks = (N + ORA_NCHUNK - 1) / ORA_NCHUNK;
    int64_t ntask = M * nchunks;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
        int64_t m = t / nchunks;
        int64_t n0 = (t % nchunks) * ORA_NCHUNK;
        int64_t n1 = n0 + ORA_NCHUNK < N ? n0 + ORA_NCHUNK : N;
        double* c = C + m * ldc;
        double* s = S + m * ldc;
        for (int64_t n = n0; n < n1; ++n) {
            c[n] = 0.0;
            s[n] = 0.0;
        }
        double e4m3[256], e2m1[16];            /* the decoders' values of every code */
        for (int q = 0; q < 256; ++q)
            e4m3[q] = ora_dec_e4m3fn((uint8_t)q);
        for (int q = 0; q < 16; ++q)
            e2m1[q] = ora_dec_e2m1((uint8_t)q);
        for (int64_t k = 0; k < K; ++k) {
            double a = ora_dec_bf16(A[m * lda + k]);
            const uint8_t* brow = Bq + k * ldbq;
            const uint8_t* srow = sB + (k / 32) * ldsb;
            for (int64_t n = n0; n < n1; ++n) {
                uint8_t code = (uint8_t)((brow[n / 2] >> (4 * (n & 1))) & 15);
                double b = e2m1[code] * e4m3[srow[n]];
                double p = a * b;
                c[n] += p;
                s[n] += fabs(p);
            }
        }
    }
}

/* ------------------------------------------------------- decode attention */

/* Decode attention: one query token per sequence attends to the first
 * lens[b] cached keys of its sequence.  The pages name this operation (the
 * dual-kernel decode attention of the QbitAI article on V4's batch
 * invariance, the part on split-KV, and section 4.1 of the lshu.cn article)
 * but print no formula, so this is the textbook scaled dot-product attention
 * (Vaswani et al. 2017, equation 1) with grouped-query heads (Ainslie et al.
 * 2023): query head h reads KV head h / G, G = Hq / Hkv.
 *
 *   z_j = scale * sum_d q[d] * k_j[d]             j < L = lens[b]
 *   w_j = exp(z_j - max_i z_i) / sum_i exp(z_i - max_i z_i)
 *   o[d] = sum_j w_j * v_j[d]
 *
 * Layouts: Q and O [B][Hq][D]; K and V [B][Hkv][Lmax][D]; all bf16 codes,
 * row-major.  O is returned in binary64.  Optional outputs (NULL to skip):
 * W [B][Hq][Lmax] the normalised weights w_j (0 for j >= L) and
 * A [B][Hq][Lmax] the absolute dot products sum_d |q[d] * k_j[d]|, which
 * scale the rounding error of a binary32 score.  L = 0 gives o = 0.
 * Subtracting the maximum does not change w_j; it only keeps exp in range. */
void ora_decode_attn(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Lmax,
                     const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                     const int32_t* lens, double scale,
                     double* O, double* W, double* A)
{
    int64_t G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < B * Hq; ++t) {
        int64_t b = t / Hq, h = t % Hq, kvh = h / G;
        int64_t L = lens[b];
        const uint16_t* q = Q + t * D;
        const uint16_t* kb = K + (b * Hkv + kvh) * Lmax * D;
        const uint16_t* vb = V + (b * Hkv + kvh) * Lmax * D;
        double* o = O + t * D;
        double* w = W ? W + t * Lmax : NULL;
        double* a = A ? A + t * Lmax : NULL;
        double s_stack[64];
        double* s = L <= 64 ? s_stack : (double*)malloc((size_t)L * sizeof(double));
        double smax = -INFINITY, den = 0.0;
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        if (w)
            for (int64_t j = 0; j < Lmax; ++j)
                w[j] = 0.0;
        if (a)
            for (int64_t j = 0; j < Lmax; ++j)
                a[j] = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double p = ora_dec_bf16(q[d]) * ora_dec_bf16(kb[j * D + d]);
                acc += p;
                aabs += fabs(p);
            }
            s[j] = scale * acc;
            if (a)
                a[j] = aabs;
            if (s[j] > smax)
                smax = s[j];
        }
        for (int64_t j = 0; j < L; ++j) {
            s[j] = exp(s[j] - smax);
            den += s[j];
        }
        for (int64_t j = 0; j < L; ++j) {
            double wj = s[j] / den;
            if (w)
                w[j] = wj;
            for (int64_t d = 0; d < D; ++d)
                o[d] += wj * ora_dec_bf16(vb[j * D + d]);
        }
        if (s != s_stack)
            free(s);
    }
}
