// gemm_skinny.hpp -- narrow-M W4A8 kernel for gfx950 (decode-like shapes).
//
// For M <= 16 the product is bound by reading the packed weights B once from
// HBM.  The kernel streams B straight from global memory into registers
// (16-byte vector loads, no LDS staging), unpacks the nibbles and contracts
// them with v_mfma_i32_16x16x64_i8, B playing the MFMA's 16-row operand and
// the (zero-padded) rows of A its 16-column operand -- the w4a8 page's kernel
// likewise puts the dequantised B first and produces C^T.
//
// Work split: workgroup = KW waves sharing one strip of FN*16 rows of B; wave
// w covers the w-th slice of K.  The KW partial 16 x (FN*16) tiles are summed
// through LDS (exact integer sums, fixed order) and the workgroup writes its
// strip of C.  A (at most 16 x K bytes) is read through the caches by every
// strip.
//
// Requirements (checked on the host): M <= 16, K % 32 == 0, 16-byte aligned
// bases, N, K < 2^31, k_per_wave a multiple of 128.
#pragma once

#include "device_common.hpp"

namespace lpgemm {

template <int FN, int KW>
__global__ __launch_bounds__(64 * KW) void gemm_w4a8_skinny_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B, int32_t *__restrict__ C, int M,
    int N, int K, int k_per_wave)
{
    __shared__ i32x4 red[KW][FN][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;     // k group this lane feeds
    const int r16 = lane & 15;   // operand row
    const int n_strip = blockIdx.x * (FN * 16);

    const int64_t ldb = (int64_t)K / 2;
    const int k_begin = wave * k_per_wave;
    const int k_end = min(K, k_begin + k_per_wave);

    const bool a_row_ok = r16 < M;
    const int8_t *arow = A + (int64_t)(a_row_ok ? r16 : 0) * K;
    const uint8_t *brow[FN];
    bool b_row_ok[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int n = n_strip + fn * 16 + r16;
        b_row_ok[fn] = n < N;
        brow[fn] = B + (int64_t)(b_row_ok[fn] ? n : 0) * ldb;
    }

    i32x4 acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = i32x4{0, 0, 0, 0};

    // One step = 128 logical k: each lane reads 16 packed bytes (32 k) of each
    // of its B rows and the matching 32 int8 of its A row.
    for (int k = k_begin; k < k_end; k += 128) {
        const int kl = k + 32 * g;  // first logical k of this lane's slice
        const bool k_ok = kl < K;
        i32x4 q[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            q[fn] = (k_ok && b_row_ok[fn]) ? load16(brow[fn] + kl / 2) : i32x4{0, 0, 0, 0};
        const bool a_ok = k_ok && a_row_ok;
        const i32x4 a_lo = a_ok ? load16(arow + kl) : i32x4{0, 0, 0, 0};
        const i32x4 a_hi = a_ok ? load16(arow + kl + 16) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            i32x4 b_lo, b_hi;
            unpack_chunk<true>(q[fn], b_lo, b_hi);
            acc[fn] = mfma_16x16x64(b_lo, a_lo, acc[fn]);
            acc[fn] = mfma_16x16x64(b_hi, a_hi, acc[fn]);
        }
    }

#pragma unroll
    for (int fn = 0; fn < FN; ++fn) red[wave][fn][lane] = acc[fn];
    __syncthreads();

    // Sum the KW partial tiles; thread t finishes lane (t % 64) of strip block
    // fn = t / 64 (and further blocks when FN > KW).
    for (int e = threadIdx.x; e < FN * 64; e += 64 * KW) {
        const int fn = e >> 6, l = e & 63;
        i32x4 s = red[0][fn][l];
#pragma unroll
        for (int w = 1; w < KW; ++w) s += red[w][fn][l];
        s >>= 4;
        const int m = l & 15;
        const int n = n_strip + fn * 16 + 4 * (l >> 4);
        if (m >= M) continue;
        int32_t *crow = C + (int64_t)m * N;
        if ((N % 4) == 0 && n + 3 < N) {
            *reinterpret_cast<i32x4 *>(crow + n) = s;
        } else {
            if (n + 0 < N) crow[n + 0] = s.x;
            if (n + 1 < N) crow[n + 1] = s.y;
            if (n + 2 < N) crow[n + 2] = s.z;
            if (n + 3 < N) crow[n + 3] = s.w;
        }
    }
}

}  // namespace lpgemm
