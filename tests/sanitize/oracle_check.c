/*
 * Drives every entry point of the C oracle (oracle/lpgemm_oracle.c) on small
 * random and edge-case inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: out-of-bounds accesses, overflows and other
 * undefined behaviour in the oracle abort the run.  Light consistency checks
 * (element-wise calls against whole products, W4A8 against int4 x int4 where A
 * fits 4 bits, pack/unpack round trips) make sure every path runs to the end.
 * Exit status 0 when all of it passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
void oracle_set_num_threads(int n);
int oracle_unpack_int4(const uint8_t *packed, int64_t rows, int64_t K, int8_t *out);
int oracle_pack_int4(const int8_t *logical, int64_t rows, int64_t K, uint8_t *out);
int oracle_gemm_i4i4(const uint8_t *Ap, const uint8_t *Bp, int64_t M, int64_t N, int64_t K, int32_t *C);
int oracle_gemm_w4a8(const int8_t *A, const uint8_t *Bp, int64_t M, int64_t N, int64_t K, int32_t *C);
int oracle_gemm_i4i4_at(const uint8_t *Ap, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count, int32_t *out);
int oracle_gemm_w4a8_at(const int8_t *A, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count, int32_t *out);
int oracle_scaled_epilogue(const int32_t *C, const float *scale_a, const float *scale_b, int64_t M,
                           int64_t N, int fmt, double *out);
int oracle_fp8_e4m3_decode(const uint8_t *codes, int64_t n, double *out);
int oracle_fp8_e4m3_encode(const double *x, int64_t n, uint8_t *out);
int oracle_gemm_fp8(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K, double *C,
                    double *Cabs);
int oracle_gemm_blockscaled(int variant, const uint8_t *A, const uint8_t *Bp, const float *SFA,
                            const float *SFB, int64_t M, int64_t N, int64_t K, int64_t g, int fmt,
                            double *out);
int oracle_fp8_e5m2_decode(const uint8_t *codes, int64_t n, double *out);
int oracle_fp8_e5m2_encode(const double *x, int64_t n, uint8_t *out);
int oracle_gemm_fp8_e5m2(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                         double *C, double *Cabs);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static void *alloc(size_t n) { return malloc(n ? n : 1); }

static void gemms(int64_t M, int64_t N, int64_t K)
{
    const int64_t h = K / 2;
    uint8_t *Ap = alloc((size_t)(M * h)), *Bp = alloc((size_t)(N * h));
    int8_t *A8 = alloc((size_t)(M * K)), *Al = alloc((size_t)(M * K));
    int32_t *C = alloc((size_t)(M * N) * 4), *C2 = alloc((size_t)(M * N) * 4);
    for (int64_t i = 0; i < M * h; ++i) Ap[i] = (uint8_t)next();
    for (int64_t i = 0; i < N * h; ++i) Bp[i] = (uint8_t)next();
    for (int64_t i = 0; i < M * K; ++i) A8[i] = (int8_t)next();
    CHECK(oracle_gemm_i4i4(Ap, Bp, M, N, K, C) == 0);
    CHECK(oracle_gemm_w4a8(A8, Bp, M, N, K, C2) == 0);
    /* element-wise calls agree with the whole products */
    int64_t ms[7], ns[7];
    int32_t at[7];
    const int64_t cnt = M && N ? 7 : 0;
    for (int i = 0; i < cnt; ++i) {
        ms[i] = (int64_t)(next() % (uint64_t)M);
        ns[i] = (int64_t)(next() % (uint64_t)N);
    }
    CHECK(oracle_gemm_i4i4_at(Ap, Bp, M, N, K, ms, ns, cnt, at) == 0);
    for (int i = 0; i < cnt; ++i) CHECK(at[i] == C[ms[i] * N + ns[i]]);
    CHECK(oracle_gemm_w4a8_at(A8, Bp, M, N, K, ms, ns, cnt, at) == 0);
    for (int i = 0; i < cnt; ++i) CHECK(at[i] == C2[ms[i] * N + ns[i]]);
    /* W4A8 with A's values in [-8, 7] equals int4 x int4 of A packed */
    CHECK(oracle_unpack_int4(Ap, M, K, Al) == 0);
    CHECK(oracle_gemm_w4a8(Al, Bp, M, N, K, C2) == 0);
    CHECK(memcmp(C, C2, (size_t)(M * N) * 4) == 0);
    uint8_t *Ap2 = alloc((size_t)(M * h));
    CHECK(oracle_pack_int4(Al, M, K, Ap2) == 0);
    CHECK(memcmp(Ap, Ap2, (size_t)(M * h)) == 0);
    /* the scaled epilogue in every format */
    float *sa = alloc((size_t)M * 4), *sb = alloc((size_t)N * 4);
    double *D = alloc((size_t)(M * N) * 8);
    for (int64_t i = 0; i < M; ++i) sa[i] = ldexpf((float)(int32_t)next(), -40);
    for (int64_t i = 0; i < N; ++i) sb[i] = ldexpf((float)(int32_t)next(), -38);
    for (int fmt = 0; fmt <= 2; ++fmt) CHECK(oracle_scaled_epilogue(C, sa, sb, M, N, fmt, D) == 0);
    CHECK(oracle_scaled_epilogue(C, sa, sb, M, N, 3, D) != 0);   /* unknown format */
    /* per-K-block scales, g = 32 and 128 (ragged last block), every format */
    for (int64_t g = 32; g <= 128; g *= 4) {
        const int64_t nb = (K + g - 1) / g;
        float *sfa = alloc((size_t)(M * nb) * 4), *sfb = alloc((size_t)(N * nb) * 4);
        for (int64_t i = 0; i < M * nb; ++i) sfa[i] = ldexpf((float)(int32_t)next(), -40);
        for (int64_t i = 0; i < N * nb; ++i) sfb[i] = ldexpf((float)(int32_t)next(), -38);
        for (int fmt = 0; fmt <= 2; ++fmt) {
            CHECK(oracle_gemm_blockscaled(0, Ap, Bp, sfa, sfb, M, N, K, g, fmt, D) == 0);
            CHECK(oracle_gemm_blockscaled(1, (const uint8_t *)A8, Bp, sfa, sfb, M, N, K, g, fmt, D) == 0);
        }
        CHECK(oracle_gemm_blockscaled(2, Ap, Bp, sfa, sfb, M, N, K, g, 0, D) != 0);   /* unknown variant */
        free(sfa); free(sfb);
    }
    free(Ap); free(Bp); free(A8); free(Al); free(C); free(C2); free(Ap2); free(sa); free(sb); free(D);
}

static void fp8(int64_t M, int64_t N, int64_t K)
{
    uint8_t *A = alloc((size_t)(M * K)), *B = alloc((size_t)(N * K));
    for (int64_t i = 0; i < M * K; ++i) { A[i] = (uint8_t)next(); if ((A[i] & 0x7F) == 0x7F) A[i] &= 0xF8; }
    for (int64_t i = 0; i < N * K; ++i) { B[i] = (uint8_t)next(); if ((B[i] & 0x7F) == 0x7F) B[i] &= 0xF8; }
    double *C = alloc((size_t)(M * N) * 8), *Cabs = alloc((size_t)(M * N) * 8);
    CHECK(oracle_gemm_fp8(A, B, M, N, K, C, Cabs) == 0);
    uint8_t *enc = alloc((size_t)(M * N));
    CHECK(oracle_fp8_e4m3_encode(C, M * N, enc) == 0);
    /* e5m2: every byte is a code (infinities and NaNs included) */
    for (int64_t i = 0; i < M * K; ++i) A[i] = (uint8_t)next();
    for (int64_t i = 0; i < N * K; ++i) B[i] = (uint8_t)next();
    CHECK(oracle_gemm_fp8_e5m2(A, B, M, N, K, C, Cabs) == 0);
    CHECK(oracle_fp8_e5m2_encode(C, M * N, enc) == 0);
    free(A); free(B); free(C); free(Cabs); free(enc);
}

int main(void)
{
    oracle_set_num_threads(2);
    CHECK(oracle_num_threads() >= 1);
    /* all 256 codes and bytes */
    uint8_t all[256], back[256];
    double v[256];
    for (int i = 0; i < 256; ++i) all[i] = (uint8_t)i;
    CHECK(oracle_fp8_e4m3_decode(all, 256, v) == 0);
    for (int i = 0; i < 256; ++i) if (isnan(v[i])) v[i] = 0.0;
    CHECK(oracle_fp8_e4m3_encode(v, 256, back) == 0);
    CHECK(oracle_fp8_e5m2_decode(all, 256, v) == 0);
    CHECK(oracle_fp8_e5m2_encode(v, 256, back) == 0);
    int8_t lg[512];
    CHECK(oracle_unpack_int4(all, 1, 512, lg) == 0);
    CHECK(oracle_pack_int4(lg, 1, 512, back) == 0);
    CHECK(memcmp(all, back, 256) == 0);
    /* shapes: ragged, empty, K = 0, one element, a few tiles' worth */
    const int64_t shapes[][3] = {{1, 1, 2}, {3, 5, 2}, {17, 33, 34}, {37, 53, 86}, {0, 4, 8},
                                 {4, 0, 8}, {5, 7, 0}, {64, 64, 256}, {129, 31, 1030}, {2, 3, 4098}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        gemms(shapes[i][0], shapes[i][1], shapes[i][2]);
        fp8(shapes[i][0], shapes[i][1], shapes[i][2] + 1);
    }
    /* argument errors are reported, not undefined */
    int32_t c1[1];
    uint8_t b1[2] = {0, 0};
    CHECK(oracle_gemm_i4i4(b1, b1, 1, 1, 3, c1) != 0);     /* odd K */
    CHECK(oracle_gemm_i4i4(b1, b1, -1, 1, 2, c1) != 0);    /* negative size */
    CHECK(oracle_pack_int4(lg, 1, 3, back) != 0);
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    else printf("oracle sanitizer run: all checks passed\n");
    return failures ? 1 : 0;
}
