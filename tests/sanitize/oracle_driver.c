/* Runs every function of the C oracle on small inputs held in buffers of
 * exactly the extents the documented layouts imply (so AddressSanitizer
 * reports any read or write past them), with row pitches wider than a row,
 * ragged shapes and the degenerate sizes, under UndefinedBehaviorSanitizer.
 * Values are small integers times powers of two, so every sum is exact in
 * binary64 and the result can be checked against a direct count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double ora_dec_bf16(uint16_t h);
double ora_dec_e4m3fn(uint8_t q);
double ora_dec_e2m1(uint8_t nib);
double ora_dec_e8m0(uint8_t e);
uint16_t ora_rne_bf16(double x);
void ora_round_bf16(int64_t n, const double* x, uint16_t* out);
int ora_num_threads(void);
void ora_set_num_threads(int n);
void ora_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                   const uint16_t* B, int64_t ldb, double* C, double* S, int64_t ldc);
void ora_gemm_fp8bs(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const float* sA, int64_t ldsa, const uint8_t* B, int64_t ldb, const float* sB,
                    int64_t ldsb, double* C, double* S, int64_t ldc);
void ora_gemm_w4a8(int64_t M, int64_t N, int64_t K, const uint8_t* qA, int64_t lda,
                   const float* sA, int64_t ldsa, const uint8_t* Bq, int64_t ldbq,
                   const uint8_t* sE, int64_t ldse, double* C, double* S, int64_t ldc);
void ora_gemm_fp4w(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                   const uint8_t* Bq, int64_t ldbq, const uint8_t* sB, int64_t ldsb, double* C,
                   double* S, int64_t ldc);
void ora_decode_attn(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Lmax,
                     const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* lens,
                     double scale, double* O, double* W, double* A);

static int failures = 0;
static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 11);
}

static void fail(const char* what)
{
    fprintf(stderr, "FAIL %s\n", what);
    ++failures;
}

/* the bf16 code of a small integer (|v| <= 256 is exact in 8 bits) */
static uint16_t bf16_of(int v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void decoders(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        double d = ora_dec_bf16((uint16_t)h);
        uint16_t back = ora_rne_bf16(d);
        if (isnan(d) ? back != 0x7FC0 : back != h)
            fail("bf16 decode / round trip");
    }
    for (int q = 0; q < 256; ++q) {
        double v = ora_dec_e4m3fn((uint8_t)q);
        if ((q & 0x7F) == 0x7F ? !isnan(v) : (isnan(v) || fabs(v) > 448.0))
            fail("e4m3fn decode");
        double e = ora_dec_e8m0((uint8_t)q);
        if (q == 255 ? !isnan(e) : e != ldexp(1.0, q - 127))
            fail("e8m0 decode");
    }
    for (int n = 0; n < 16; ++n)
        if (fabs(ora_dec_e2m1((uint8_t)n)) > 6.0)
            fail("e2m1 decode");
    const double special[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e300, -1e300, 1e-300,
                              ldexp(1.0, -133), ldexp(1.0, -134), ldexp(3.0, -134)};
    uint16_t out[sizeof special / sizeof special[0]];
    ora_round_bf16((int64_t)(sizeof special / sizeof special[0]), special, out);
    if (out[0] != 0 || out[1] != 0x8000 || out[2] != 0x7F80 || out[3] != 0xFF80 ||
        out[4] != 0x7FC0 || out[5] != 0x7F80 || out[6] != 0xFF80 || out[7] != 0 || out[8] != 1 ||
        out[9] != 0 || out[10] != 2)
        fail("bf16 rounding of special values");
}

static void* take(size_t n) { return malloc(n ? n : 1); }

static void gemm_bf16(int64_t M, int64_t N, int64_t K)
{
    const int64_t lda = K + 3, ldb = N + 5, ldc = N + 2;
    uint16_t* A = take((size_t)((M ? M - 1 : 0) * lda + K) * 2);
    uint16_t* B = take((size_t)((K ? K - 1 : 0) * ldb + N) * 2);
    int* a = take((size_t)(M * K) * sizeof(int));
    int* b = take((size_t)(K * N) * sizeof(int));
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            A[i * lda + k] = bf16_of(a[i * K + k] = (int)(next() % 17) - 8);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            B[k * ldb + j] = bf16_of(b[k * N + j] = (int)(next() % 17) - 8);
    size_t nc = (size_t)((M ? M - 1 : 0) * ldc + N);
    double* C = take(nc * sizeof(double));
    double* S = take(nc * sizeof(double));
    ora_gemm_bf16(M, N, K, A, lda, B, ldb, C, S, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            long c = 0, s = 0;
            for (int64_t k = 0; k < K; ++k) {
                long p = (long)a[i * K + k] * b[k * N + j];
                c += p;
                s += labs(p);
            }
            if (C[i * ldc + j] != (double)c || S[i * ldc + j] != (double)s)
                fail("bf16 GEMM sum");
        }
    free(A); free(B); free(a); free(b); free(C); free(S);
}

/* e4m3fn code of +-v for v in {0, 1, 2, 4}: exponent field 7 + log2 v */
static uint8_t e4m3_of(int v)
{
    int a = abs(v);
    uint8_t q = a == 0 ? 0 : (uint8_t)((7 + (a == 1 ? 0 : a == 2 ? 1 : 2)) << 3);
    return (uint8_t)(v < 0 ? q | 0x80 : q);
}

static void gemm_fp8(int64_t M, int64_t N, int64_t K)
{
    const int64_t kb = K / 128, nb = (N + 127) / 128;
    const int64_t lda = K + 16, ldb = N + 7, ldsa = kb + 1, ldsb = nb + 2, ldc = N + 1;
    uint8_t* A = take((size_t)((M ? M - 1 : 0) * lda + K));
    uint8_t* B = take((size_t)((K ? K - 1 : 0) * ldb + N));
    float* sA = take((size_t)((M ? M - 1 : 0) * ldsa + kb) * sizeof(float));
    float* sB = take((size_t)((kb ? kb - 1 : 0) * ldsb + nb) * sizeof(float));
    static const int vals[] = {0, 1, -1, 2, -2, 4, -4};
    int* a = take((size_t)(M * K) * sizeof(int));
    int* b = take((size_t)(K * N) * sizeof(int));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k)
            A[i * lda + k] = e4m3_of(a[i * K + k] = vals[next() % 7]);
        for (int64_t t = 0; t < kb; ++t)
            sA[i * ldsa + t] = (float)(1 << (next() % 3));
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            B[k * ldb + j] = e4m3_of(b[k * N + j] = vals[next() % 7]);
    for (int64_t t = 0; t < kb; ++t)
        for (int64_t u = 0; u < nb; ++u)
            sB[t * ldsb + u] = (float)(1 << (next() % 3));
    size_t nc = (size_t)((M ? M - 1 : 0) * ldc + N);
    double* C = take(nc * sizeof(double));
    double* S = take(nc * sizeof(double));
    ora_gemm_fp8bs(M, N, K, A, lda, sA, ldsa, B, ldb, sB, ldsb, C, S, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            long c = 0;
            for (int64_t k = 0; k < K; ++k)
                c += (long)a[i * K + k] * b[k * N + j] * (long)sA[i * ldsa + k / 128] *
                     (long)sB[(k / 128) * ldsb + j / 128];
            if (C[i * ldc + j] != (double)c)
                fail("fp8 GEMM sum");
        }
    free(A); free(B); free(sA); free(sB); free(a); free(b); free(C); free(S);
}

static void gemm_fp4(int64_t M, int64_t N, int64_t K)
{
    const int64_t lda = K + 1, ldbq = N / 2 + 3, ldsb = N + 4, ldc = N + 3;
    uint16_t* A = take((size_t)((M ? M - 1 : 0) * lda + K) * 2);
    uint8_t* Bq = take((size_t)((K ? K - 1 : 0) * ldbq + N / 2));
    uint8_t* sB = take((size_t)((K / 32 ? K / 32 - 1 : 0) * ldsb + N));
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            A[i * lda + k] = bf16_of((int)(next() % 9) - 4);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j)
            Bq[k * ldbq + j] = (uint8_t)next();
    for (int64_t t = 0; t < K / 32; ++t)
        for (int64_t j = 0; j < N; ++j)
            sB[t * ldsb + j] = e4m3_of(1 << (next() % 3));
    size_t nc = (size_t)((M ? M - 1 : 0) * ldc + N);
    double* C = take(nc * sizeof(double));
    double* S = take(nc * sizeof(double));
    ora_gemm_fp4w(M, N, K, A, lda, Bq, ldbq, sB, ldsb, C, S, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            if (!(S[i * ldc + j] >= fabs(C[i * ldc + j])))
                fail("fp4 GEMM bound");
    free(A); free(Bq); free(sB); free(C); free(S);
}

static void gemm_w4a8(int64_t M, int64_t N, int64_t K)
{
    const int64_t lda = K + 16, ldsa = K / 128 + 1, ldbq = N / 2 + 1, ldse = N + 2, ldc = N;
    uint8_t* A = take((size_t)((M ? M - 1 : 0) * lda + K));
    float* sA = take((size_t)((M ? M - 1 : 0) * ldsa + K / 128) * sizeof(float));
    uint8_t* Bq = take((size_t)((K ? K - 1 : 0) * ldbq + N / 2));
    uint8_t* sE = take((size_t)((K / 32 ? K / 32 - 1 : 0) * ldse + N));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k)
            A[i * lda + k] = e4m3_of((int)(next() % 5) - 2 == 0 ? 0 : 1);
        for (int64_t t = 0; t < K / 128; ++t)
            sA[i * ldsa + t] = 0.5f;
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j)
            Bq[k * ldbq + j] = (uint8_t)next();
    for (int64_t t = 0; t < K / 32; ++t)
        for (int64_t j = 0; j < N; ++j)
            sE[t * ldse + j] = (uint8_t)(120 + next() % 10);
    size_t nc = (size_t)((M ? M - 1 : 0) * ldc + N);
    double* C = take(nc * sizeof(double));
    double* S = take(nc * sizeof(double));
    ora_gemm_w4a8(M, N, K, A, lda, sA, ldsa, Bq, ldbq, sE, ldse, C, S, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            if (!(S[i * ldc + j] >= fabs(C[i * ldc + j])))
                fail("w4a8 GEMM bound");
    free(A); free(sA); free(Bq); free(sE); free(C); free(S);
}

static void attention(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax)
{
    const int64_t D = 128;
    uint16_t* Q = take((size_t)(B * Hq * D) * 2);
    uint16_t* K = take((size_t)(B * Hkv * Lmax * D) * 2);
    uint16_t* V = take((size_t)(B * Hkv * Lmax * D) * 2);
    int32_t* lens = take((size_t)B * sizeof(int32_t));
    for (int64_t i = 0; i < B * Hq * D; ++i)
        Q[i] = bf16_of((int)(next() % 5) - 2);
    for (int64_t i = 0; i < B * Hkv * Lmax * D; ++i) {
        K[i] = bf16_of((int)(next() % 5) - 2);
        V[i] = bf16_of((int)(next() % 9) - 4);
    }
    for (int64_t b = 0; b < B; ++b)
        lens[b] = (int32_t)(b == 0 ? 0 : b == 1 ? Lmax : (int64_t)(next() % (uint32_t)(Lmax + 1)));
    double* O = take((size_t)(B * Hq * D) * sizeof(double));
    double* W = take((size_t)(B * Hq * Lmax) * sizeof(double));
    double* A = take((size_t)(B * Hq * Lmax) * sizeof(double));
    ora_decode_attn(B, Hq, Hkv, D, Lmax, Q, K, V, lens, 0.0883883476, O, W, A);
    for (int64_t t = 0; t < B * Hq; ++t) {
        double sum = 0.0;
        for (int64_t j = 0; j < Lmax; ++j)
            sum += W[t * Lmax + j];
        int64_t L = lens[t / Hq];
        if (L == 0 ? sum != 0.0 : fabs(sum - 1.0) > 1e-12)
            fail("attention weights sum");
        for (int64_t d = 0; d < D; ++d)
            if (fabs(O[t * D + d]) > 4.0 + 1e-12)
                fail("attention output outside the values' hull");
    }
    ora_decode_attn(B, Hq, Hkv, D, Lmax, Q, K, V, lens, 0.5, O, NULL, NULL);
    free(Q); free(K); free(V); free(lens); free(O); free(W); free(A);
}

int main(void)
{
    decoders();
    const int threads[] = {1, 3};
    for (int t = 0; t < 2; ++t) {
        ora_set_num_threads(threads[t]);
        if (ora_num_threads() < 1)
            fail("thread count");
        gemm_bf16(0, 5, 7);
        gemm_bf16(3, 0, 7);
        gemm_bf16(4, 6, 0);
        gemm_bf16(17, 301, 45);
        gemm_fp8(0, 9, 128);
        gemm_fp8(5, 130, 0);
        gemm_fp8(7, 259, 384);
        gemm_fp4(0, 8, 32);
        gemm_fp4(6, 70, 96);
        gemm_w4a8(5, 34, 256);
        attention(3, 8, 2, 70);
        attention(2, 4, 4, 5);
    }
    ora_set_num_threads(0);
    if (failures) {
        fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
