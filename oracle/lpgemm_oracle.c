/*
 * lpgemm_oracle.c -- plain CPU oracle for the low-precision integer GEMM
 *
 *     C[M,N] = A[M,K] . B[N,K]^T      (exact integer result, stored as int32)
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no code, header, table or constant with the GPU library: it is the
 * written-out definition the GPU results are compared against, bit for bit.
 *
 * Sources (web pages; cited by title and the passage used):
 *  [int4-gemm]  tilelang pull request "[CUDA] Support int4 T.gemm" (#2063),
 *               example "gemm_int4": matmul_nt_int4 -- A[M,K] and B[N,K] int4,
 *               C[M,N] int32, T.gemm(..., transpose_B=True), i.e. C = A . B^T.
 *  [w4a8]       tilelang pull request "[Example] add w4a8 gemm kernel" (#815),
 *               review threads on torch_convert (byte j//2, nibble j%2; the
 *               vectorised rewrite: low = b & 0x0F, high = b >> 4, subtract 16
 *               when the 4-bit value is >= 8, interleave low then high),
 *               ref_program (C = A . B^T of int8 A and the unpacked B; the
 *               reviewers ask for an integer, not a float, reference) and the
 *               kernel's in_dtype int8 / accum_dtype int32.
 *  [tutorial]   TileLang tutorial, chapter 14 section 5 "low_precision_gemm.py":
 *               matmul_int4 (int4 operands, int32 accumulator, two nibbles per
 *               byte) and pack_int4 (byte = (x[2j] & 0xF) | ((x[2j+1] & 0xF) << 4),
 *               last dimension must be even).
 *
 * Every routine is the plain definition: unpack each operand once into int8,
 * then a triple loop m, n, k accumulating in int64.  The outer m loop is split
 * across OpenMP threads; nothing else is reordered, blocked or fused.  The sum
 * is checked to fit int32 before it is stored (the pages store int32).
 *
 * Return codes: 0 ok, 1 bad argument (negative size, odd K, null pointer),
 * 2 a result outside int32, 3 out of host memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_RANGE 2
#define ORACLE_ERR_NOMEM 3

/* The 4-bit field holding logical element k of a packed row: element k lives
 * in byte k/2; even k in the low nibble, odd k in the high nibble ([w4a8]
 * torch_convert indexes byte j//2, nibble j%2; [tutorial] pack_int4 puts
 * x[0::2] low and x[1::2] high).  The byte is read as unsigned. */
static unsigned nibble_of(const uint8_t *row, int64_t k)
{
    uint8_t byte = row[k / 2];
    return (k % 2 == 0) ? (unsigned)(byte & 0x0Fu) : (unsigned)(byte >> 4);
}

/* Two's-complement value of a 4-bit field: subtract 16 when the field is 8 or
 * more ([w4a8], the vectorised torch_convert). */
static int int4_value(unsigned field)
{
    return (int)field - (field >= 8u ? 16 : 0);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the later calls (timing only; the results do not depend on it). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Unpack rows x K logical int4 from packed bytes [rows][K/2] into int8 [rows][K]. */
int oracle_unpack_int4(const uint8_t *packed, int64_t rows, int64_t K, int8_t *out)
{
    if (rows < 0 || K < 0 || K % 2 != 0) return ORACLE_ERR_ARG;
    if (rows * K > 0 && (packed == NULL || out == NULL)) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t *src = packed + r * (K / 2);
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = (int8_t)int4_value(nibble_of(src, k));
    }
    return ORACLE_OK;
}

/* Pack rows x K logical int4 (held as int8) into bytes [rows][K/2]:
 * byte j = (x[2j] & 0xF) | ((x[2j+1] & 0xF) << 4)   ([tutorial] pack_int4).
 * Like the page's packer it keeps only the low four bits of each value. */
int oracle_pack_int4(const int8_t *logical, int64_t rows, int64_t K, uint8_t *out)
{
    if (rows < 0 || K < 0 || K % 2 != 0) return ORACLE_ERR_ARG;
    if (rows * K > 0 && (logical == NULL || out == NULL)) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        const int8_t *x = logical + r * K;
        for (int64_t j = 0; j < K / 2; ++j) {
            unsigned even = (unsigned)(uint8_t)x[2 * j] & 0x0Fu;
            unsigned odd = (unsigned)(uint8_t)x[2 * j + 1] & 0x0Fu;
            out[r * (K / 2) + j] = (uint8_t)(even | (odd << 4));
        }
    }
    return ORACLE_OK;
}

/* C[m][n] = sum_k a[m][k] * b[n][k] over int8 rows, int64 accumulation. */
static int gemm_rows_int8(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K,
                          int32_t *C)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        const int8_t *arow = a + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *brow = b + n * K;
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)arow[k] * (int64_t)brow[k];
            if (sum < INT32_MIN || sum > INT32_MAX) bad = 1;
            C[m * N + n] = (int32_t)sum;
        }
    }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

static int check_dims(int64_t M, int64_t N, int64_t K)
{
    return (M < 0 || N < 0 || K < 0 || K % 2 != 0) ? ORACLE_ERR_ARG : ORACLE_OK;
}

/* int4 x int4: A packed [M][K/2], B packed [N][K/2], C int32 [M][N]
 * ([int4-gemm] matmul_nt_int4; [tutorial] matmul_int4). */
int oracle_gemm_i4i4(const uint8_t *Ap, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                     int32_t *C)
{
    int rc = check_dims(M, N, K);
    if (rc) return rc;
    if (M * N == 0) return ORACLE_OK;
    if (C == NULL || (K > 0 && (Ap == NULL || Bp == NULL))) return ORACLE_ERR_ARG;
    int8_t *a = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    int8_t *b = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
    if (a == NULL || b == NULL) { free(a); free(b); return ORACLE_ERR_NOMEM; }
    oracle_unpack_int4(Ap, M, K, a);
    oracle_unpack_int4(Bp, N, K, b);
    rc = gemm_rows_int8(a, b, M, N, K, C);
    free(a);
    free(b);
    return rc;
}

/* W4A8: A int8 [M][K], B packed int4 [N][K/2], C int32 [M][N]
 * ([w4a8] ref_program: A . B^T with B unpacked by torch_convert). */
int oracle_gemm_w4a8(const int8_t *A, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                     int32_t *C)
{
    int rc = check_dims(M, N, K);
    if (rc) return rc;
    if (M * N == 0) return ORACLE_OK;
    if (C == NULL || (K > 0 && (A == NULL || Bp == NULL))) return ORACLE_ERR_ARG;
    int8_t *b = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
    if (b == NULL) return ORACLE_ERR_NOMEM;
    oracle_unpack_int4(Bp, N, K, b);
    rc = gemm_rows_int8(A, b, M, N, K, C);
    free(b);
    return rc;
}

/* Selected elements one by one, straight from the packed bytes: out[i] =
 * C[ms[i]][ns[i]].  For shapes too large for the full triple loop. */
int oracle_gemm_i4i4_at(const uint8_t *Ap, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count, int32_t *out)
{
    int rc = check_dims(M, N, K);
    if (rc) return rc;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) { bad |= 2; continue; }
        const uint8_t *arow = Ap + m * (K / 2);
        const uint8_t *brow = Bp + n * (K / 2);
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k)
            sum += (int64_t)int4_value(nibble_of(arow, k)) * int4_value(nibble_of(brow, k));
        if (sum < INT32_MIN || sum > INT32_MAX) bad |= 1;
        out[i] = (int32_t)sum;
    }
    if (bad & 2) return ORACLE_ERR_ARG;
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

int oracle_gemm_w4a8_at(const int8_t *A, const uint8_t *Bp, int64_t M, int64_t N, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count, int32_t *out)
{
    int rc = check_dims(M, N, K);
    if (rc) return rc;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) { bad |= 2; continue; }
        const int8_t *arow = A + m * K;
        const uint8_t *brow = Bp + n * (K / 2);
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k)
            sum += (int64_t)arow[k] * int4_value(nibble_of(brow, k));
        if (sum < INT32_MIN || sum > INT32_MAX) bad |= 1;
        out[i] = (int32_t)sum;
    }
    if (bad & 2) return ORACLE_ERR_ARG;
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* ---- per-row / per-column scaled output ---------------------------------------
 * [tutorial] gemm_blockscaled: scales SFA[m][kb], SFB[n][kb] applied per block
 * of K with fp32 accumulation and an out_dtype result.  With a single K block
 * (one scale per row of A and per row of B) and the exact integer sum C:
 *     D[m][n] = out( ((float)C[m][n] * scale_a[m]) * scale_b[n] )
 * each step in IEEE binary32 with round-to-nearest-even, then out() rounds the
 * binary32 value to the output format, nearest even.  Formats: 0 binary32,
 * 1 bfloat16 (8 significant bits, binary32's exponent range), 2 binary16
 * (11 significant bits, normal exponents -14..15, subnormals down to 2^-24).
 * The result is returned as the exact value of the rounded number, in double. */

/* Round x (a finite binary32 value held in a double) to a binary format with
 * `digits` significant bits, smallest normal exponent `emin` and largest
 * finite value `maxv`, ties to even: the written-out definition, scaling the
 * value so the format's quantum at x becomes 1 and rounding with rint (the
 * default rounding mode is nearest-even).  Values at or beyond the midpoint
 * between maxv and the next power of two overflow to infinity (the tie goes
 * to the even neighbour, which is the infinity). */
static double round_to_format(double x, int digits, int emin, double maxv)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    const double ax = fabs(x);
    int e2;
    frexp(ax, &e2);             /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;             /* ax in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;     /* subnormal range: fixed quantum */
    const double q = ldexp(1.0, e - (digits - 1));
    const double r = rint(ax / q) * q;
    const double next_pow = ldexp(1.0, (int)floor(log2(maxv)) + 1);
    const double limit = maxv + (next_pow - maxv) / 2;
    if (ax >= limit || r > maxv) return copysign(INFINITY, x);
    return copysign(r, x);
}

int oracle_scaled_epilogue(const int32_t *C, const float *scale_a, const float *scale_b,
                           int64_t M, int64_t N, int fmt, double *out)
{
    if (M < 0 || N < 0 || fmt < 0 || fmt > 2) return 1;
    if (M == 0 || N == 0) return 0;
    if (!C || !scale_a || !scale_b || !out) return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            volatile float t = (float)C[m * N + n]; /* int32 -> binary32, nearest even */
            volatile float y = t * scale_a[m];      /* binary32 multiply */
            volatile float z = y * scale_b[n];      /* binary32 multiply */
            double v = (double)z;
            if (fmt == 1)
                v = round_to_format(v, 8, -126, ldexp(255.0, 120));    /* (2 - 2^-7) * 2^127 */
            else if (fmt == 2)
                v = round_to_format(v, 11, -14, 65504.0);
            out[m * N + n] = v;
        }
    return 0;
}

/* ---- per-K-block scaled product ------------------------------------------------
 * [tutorial] gemm_blockscaled: SFA[M][ceil(K/g)] and SFB[N][ceil(K/g)] hold
 * float32 scales (g = sf_granularity_k; the page names 128 and 32), applied
 * along K one block of g at a time into a float32 accumulator, the result
 * stored as out_dtype.  The page leaves the arithmetic to another chapter; the
 * reading taken for the integer operands:
 *   block j covers k in [j g, min(K, (j+1) g)), nb = ceil(K / g) blocks;
 *   C_j = the exact integer sum of a(m,k) b(n,k) over block j;
 *   term_j = ((float)C_j * SFA[m][j]) * SFB[n][j]    (binary32, nearest even);
 *   acc = term_0, then acc = acc + term_j for j = 1, 2, ... in increasing j
 *   (binary32, nearest even); D[m][n] = out(acc), out() as for the scaled
 *   epilogue above.  K == 0 (no block) gives +0.
 * With one block (g >= K) this is the per-channel formula above.  variant 0:
 * A packed int4 [M][K/2]; variant 1: A int8 [M][K]; B packed int4 [N][K/2]. */
int oracle_gemm_blockscaled(int variant, const uint8_t *A, const uint8_t *Bp, const float *SFA,
                            const float *SFB, int64_t M, int64_t N, int64_t K, int64_t g, int fmt,
                            double *out)
{
    int rc = check_dims(M, N, K);
    if (rc) return rc;
    if ((variant != 0 && variant != 1) || g < 1 || fmt < 0 || fmt > 2) return ORACLE_ERR_ARG;
    if (M * N == 0) return ORACLE_OK;
    const int64_t nb = (K + g - 1) / g;
    if (out == NULL || (K > 0 && (A == NULL || Bp == NULL || SFA == NULL || SFB == NULL)))
        return ORACLE_ERR_ARG;
    int8_t *a = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    int8_t *b = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
    if (a == NULL || b == NULL) { free(a); free(b); return ORACLE_ERR_NOMEM; }
    if (variant == 0) {
        oracle_unpack_int4(A, M, K, a);
    } else {
        for (int64_t i = 0; i < M * K; ++i) a[i] = (int8_t)A[i];
    }
    oracle_unpack_int4(Bp, N, K, b);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        const int8_t *arow = a + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *brow = b + n * K;
            volatile float acc = 0.0f;
            for (int64_t j = 0; j < nb; ++j) {
                const int64_t k1 = (j + 1) * g < K ? (j + 1) * g : K;
                int64_t c = 0;
                for (int64_t k = j * g; k < k1; ++k)
                    c += (int64_t)arow[k] * (int64_t)brow[k];
                if (c < INT32_MIN || c > INT32_MAX) bad = 1;
                volatile float t = (float)c;               /* integer -> binary32, nearest even */
                volatile float y = t * SFA[m * nb + j];    /* binary32 multiply */
                volatile float z = y * SFB[n * nb + j];    /* binary32 multiply */
                if (j == 0)
                    acc = z;
                else
                    acc = acc + z;                         /* binary32 add */
            }
            double v = (double)acc;
            if (fmt == 1)
                v = round_to_format(v, 8, -126, ldexp(255.0, 120));
            else if (fmt == 2)
                v = round_to_format(v, 11, -14, 65504.0);
            out[m * N + n] = v;
        }
    }
    free(a);
    free(b);
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* ---- fp8 GEMM (second workload) ---------------------------------------------
 * [tutorial] gemm_fp8 (chapter 14, the fp8 example next to matmul_int4): the
 * same A[M,K] . B[N,K]^T structure (T.gemm(..., transpose_B=True)) with fp8
 * operands (determine_fp8_type: the e4m3 format), a float32 accumulator, and C
 * stored in the fp8 dtype.  The pages leave the numerics to another chapter;
 * the oracle gives the exact value of every sum (the kernel's fp32 result is
 * compared within a stated bound) and the conversion to e4m3 written out.
 *
 * E4M3 (the OCP 8-bit format without infinities, "e4m3fn"): bit 7 sign, bits
 * 6..3 exponent with bias 7, bits 2..0 mantissa.  Exponent 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; every other code is (1 + m/8) * 2^(e-7), so
 * the largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* m/8 * 2^-6 */
    else
        v = ldexp(8.0 + m, e - 10);            /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

int oracle_fp8_e4m3_decode(const uint8_t *codes, int64_t n, double *out)
{
    if (n < 0) return ORACLE_ERR_ARG;
    if (n == 0) return ORACLE_OK;
    if (!codes || !out) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
    return ORACLE_OK;
}

/* Nearest e4m3 code of x, ties to the even code (the one whose mantissa is
 * even), magnitudes beyond 448 saturating to +-448 (the finite-saturating
 * conversion); NaN -> the NaN code with x's sign.  Written as a search over the
 * 127 non-negative finite codes, which are ordered by value. */
static uint8_t e4m3_encode(double x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    const double ax = fabs(x);
    if (ax >= 448.0) return sign | 0x7E;
    int lo = 0;                                /* largest code with value <= ax */
    for (int c = 1; c <= 0x7E; ++c)
        if (e4m3_value((uint8_t)c) <= ax) lo = c;
    if (e4m3_value((uint8_t)lo) == ax) return sign | (uint8_t)lo;
    const int hi = lo + 1;                     /* next larger value (<= 0x7E) */
    const double dlo = ax - e4m3_value((uint8_t)lo), dhi = e4m3_value((uint8_t)hi) - ax;
    if (dlo < dhi) return sign | (uint8_t)lo;
    if (dhi < dlo) return sign | (uint8_t)hi;
    return sign | (uint8_t)((lo & 1) ? hi : lo);   /* tie: even mantissa */
}

int oracle_fp8_e4m3_encode(const double *x, int64_t n, uint8_t *out)
{
    if (n < 0) return ORACLE_ERR_ARG;
    if (n == 0) return ORACLE_OK;
    if (!x || !out) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
    return ORACLE_OK;
}

/* C[m][n] = sum_k a(m,k) * b(n,k) over the decoded e4m3 values, and
 * Cabs[m][n] = sum_k |a(m,k) * b(n,k)|, both in double.  Every product is a
 * multiple of 2^-18 below 2^18 in magnitude, so for K < 2^17 each running sum
 * is a multiple of 2^-18 below 2^35 and the double sums are exact.  A NaN
 * operand gives a NaN sum. */
int oracle_gemm_fp8(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                    double *C, double *Cabs)
{
    if (M < 0 || N < 0 || K < 0 || K >= ((int64_t)1 << 17)) return ORACLE_ERR_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (!C || !Cabs || (K > 0 && (!A || !B))) return ORACLE_ERR_ARG;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!a || !b) {
        free(a);
        free(b);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t i = 0; i < M * K; ++i) a[i] = e4m3_value(A[i]);
    for (int64_t i = 0; i < N * K; ++i) b[i] = e4m3_value(B[i]);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = a[m * K + k] * b[n * K + k];
                s += p;
                sa += fabs(p);
            }
            C[m * N + n] = s;
            Cabs[m * N + n] = sa;
        }
    free(a);
    free(b);
    return ORACLE_OK;
}

/* ---- fp8 GEMM with e5m2 operands ---------------------------------------------
 * [tutorial] gemm_fp8's "e4m3 / e5m2, fp32 accumulation": the same product with
 * the other fp8 dtype.
 *
 * E5M2 (the OCP 8-bit format with infinities; the top byte of an IEEE
 * binary16): bit 7 sign, bits 6..2 exponent with bias 15, bits 1..0 mantissa.
 * Exponent 0 is subnormal (m/4 * 2^-14); exponent 31 is infinity (m = 0) or
 * NaN (m != 0); every other code is (1 + m/4) * 2^(e-15), so the largest finite
 * magnitude is 1.75 * 2^15 = 57344.  Each finite value is an integer times a
 * power of two: (4 + m) * 2^(e-17), or m * 2^-16 for subnormals. */
static int e5m2_int(uint8_t c, int64_t *im, int *ie)
{
    const int e = (c >> 2) & 31, m = c & 3;
    if (e == 31) return 0;                     /* infinity or NaN */
    *im = e == 0 ? m : 4 + m;
    *ie = e == 0 ? -16 : e - 17;
    if (c & 0x80) *im = -*im;
    return 1;
}

static double e5m2_value(uint8_t c)
{
    const int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    const double v = e == 0 ? ldexp((double)m, -16) : ldexp(4.0 + m, e - 17);
    return s ? -v : v;   /* -0.0 for the code 0x80 */
}

int oracle_fp8_e5m2_decode(const uint8_t *codes, int64_t n, double *out)
{
    if (n < 0) return ORACLE_ERR_ARG;
    if (n == 0) return ORACLE_OK;
    if (!codes || !out) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e5m2_value(codes[i]);
    return ORACLE_OK;
}

/* Nearest e5m2 code of x, ties to the even code, as for any IEEE format with
 * infinities: magnitudes from the midpoint between the largest finite value and
 * 2^16 (61440) on become infinity; NaN -> S.11111.11.  A search over the 124
 * non-negative finite codes, which are ordered by value. */
static uint8_t e5m2_encode(double x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    const double ax = fabs(x);
    if (ax >= 61440.0) return sign | 0x7C;
    int lo = 0;
    for (int c = 1; c <= 0x7B; ++c)
        if (e5m2_value((uint8_t)c) <= ax) lo = c;
    if (e5m2_value((uint8_t)lo) == ax) return sign | (uint8_t)lo;
    if (lo == 0x7B) return sign | 0x7B;        /* between 57344 and 61440 */
    const int hi = lo + 1;
    const double dlo = ax - e5m2_value((uint8_t)lo), dhi = e5m2_value((uint8_t)hi) - ax;
    if (dlo < dhi) return sign | (uint8_t)lo;
    if (dhi < dlo) return sign | (uint8_t)hi;
    return sign | (uint8_t)((lo & 1) ? hi : lo);
}

int oracle_fp8_e5m2_encode(const double *x, int64_t n, uint8_t *out)
{
    if (n < 0) return ORACLE_ERR_ARG;
    if (n == 0) return ORACLE_OK;
    if (!x || !out) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e5m2_encode(x[i]);
    return ORACLE_OK;
}

/* C[m][n] = sum_k a(m,k) * b(n,k) over the decoded e5m2 values, and Cabs the
 * sum of the products' magnitudes.  Products are integers times 2^-32 below
 * 2^64 in those units; both sums are formed exactly in 128-bit integers and
 * returned as the nearest double.  An infinite or NaN operand makes the sum
 * follow IEEE arithmetic in double instead (a NaN or infinite result). */
int oracle_gemm_fp8_e5m2(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                         double *C, double *Cabs)
{
    if (M < 0 || N < 0 || K < 0 || K >= ((int64_t)1 << 17)) return ORACLE_ERR_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (!C || !Cabs || (K > 0 && (!A || !B))) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            __int128 s = 0, sa = 0;
            int finite = 1;
            for (int64_t k = 0; k < K && finite; ++k) {
                int64_t ia, ib;
                int ea, eb;
                finite = e5m2_int(A[m * K + k], &ia, &ea) && e5m2_int(B[n * K + k], &ib, &eb);
                if (!finite) break;
                const __int128 p = (__int128)(ia * ib) * ((__int128)1 << (ea + eb + 32));   /* units of 2^-32 */
                s += p;
                sa += p < 0 ? -p : p;
            }
            if (finite) {
                C[m * N + n] = ldexp((double)s, -32);
                Cabs[m * N + n] = ldexp((double)sa, -32);
            } else {
                double ds = 0.0, dsa = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double p = e5m2_value(A[m * K + k]) * e5m2_value(B[n * K + k]);
                    ds += p;
                    dsa += fabs(p);
                }
                C[m * N + n] = ds;
                Cabs[m * N + n] = dsa;
            }
        }
    return ORACLE_OK;
}
