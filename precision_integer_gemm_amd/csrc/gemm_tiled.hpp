// gemm_tiled.hpp -- block-tiled int8-MFMA GEMM for gfx950, both formats.
//
// C[M,N] = A[M,K] . B[N,K]^T ("NT": every operand row is contiguous in K, as
// in the int4 example's T.gemm(..., transpose_B=True) and the w4a8 example).
//
// Per workgroup: a BM x BN tile of C.  The K loop stages BK logical k of both
// operands per step through a double-buffered LDS ring (packed bytes stay
// packed in LDS: BK/2 bytes per 4-bit row, BK bytes per int8 row).  The next
// step's global loads (16-byte vectors, zero-filled past the edges) are in
// flight while the current step computes.  Each wave owns an FN x FM grid of
// 32x32 output blocks; per 64 k it reads one 16-byte LDS vector per block row
// and column, unpacks nibbles to x16-scaled int8 in registers, and issues
// v_mfma_i32_32x32x32_i8 twice per block.
//
// The MFMA's "row" operand is B (rows n) and its "column" operand is A (rows
// m), so the accumulator holds C^T: each lane ends with four consecutive n of
// one m, stored as one 16-byte vector.  The epilogue shifts out the x16/x256
// scale and masks m >= M and n >= N.
//
// Requirements (checked on the host): K % 32 == 0, all base pointers 16-byte
// aligned, M, N, K < 2^31.
#pragma once

#include "device_common.hpp"

namespace lpgemm {

template <int VAR, int FM, int FN, int WM, int WN, int BK>
struct TiledCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = WM * FM * 32;
    static constexpr int BN = WN * FN * 32;
    static constexpr int RA = (VAR == I4I4) ? BK / 2 : BK;  // LDS bytes per A row
    static constexpr int RB = BK / 2;                       // LDS bytes per B row
    static constexpr int CPR_A = RA / 16;                   // 16-byte chunks per row
    static constexpr int CPR_B = RB / 16;
    static constexpr int A_CHUNKS = BM * CPR_A;
    static constexpr int B_CHUNKS = BN * CPR_B;
    static constexpr int A_PER_THREAD = A_CHUNKS / kThreads;
    static constexpr int B_PER_THREAD = B_CHUNKS / kThreads;
    static constexpr int STAGE_BYTES = BM * RA + BN * RB;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int SHIFT = (VAR == I4I4) ? 8 : 4;
    static_assert(BK % 64 == 0, "BK must be a multiple of 64");
    static_assert(A_CHUNKS % kThreads == 0 && B_CHUNKS % kThreads == 0, "uneven load split");
    static_assert(CPR_A <= 16 && CPR_B <= 16, "row too long for the swizzle");
};

// XOR swizzle of 16-byte chunks inside an LDS row so that the 32 lanes that
// read the same chunk column of 32 consecutive rows spread over all banks.
template <int CPR>
__device__ __forceinline__ int swz_offset(int row, int col)
{
    constexpr int rows_per_256 = 16 / CPR;  // rows sharing one 256-byte bank line
    const int s = (row / rows_per_256) % CPR;
    return row * (CPR * 16) + ((col ^ s) * 16);
}

template <int VAR, int FM, int FN, int WM, int WN, int BK>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int32_t *__restrict__ C, int M,
    int N, int K, int tiles_n)
{
    using Cfg = TiledCfg<VAR, FM, FN, WM, WN, BK>;
    constexpr int RA = Cfg::RA, RB = Cfg::RB, CPR_A = Cfg::CPR_A, CPR_B = Cfg::CPR_B;
    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int tile_m = blockIdx.x / tiles_n;
    const int tile_n = blockIdx.x % tiles_n;
    const int m0 = tile_m * Cfg::BM;
    const int n0 = tile_n * Cfg::BN;

    const int64_t lda = (VAR == I4I4) ? (int64_t)K / 2 : (int64_t)K;  // global row bytes
    const int64_t ldb = (int64_t)K / 2;
    const int ktiles = (K + BK - 1) / BK;

    // Global -> register staging of one K step.
    i32x4 ra[Cfg::A_PER_THREAD];
    i32x4 rb[Cfg::B_PER_THREAD];

    auto load_step = [&](int kt) {
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
            const int c = tid + i * Cfg::kThreads;
            const int row = c / CPR_A, col = c % CPR_A;
            const int64_t kb = (int64_t)kt * RA + col * 16;
            const int gm = m0 + row;
            ra[i] = (gm < M && kb < lda) ? load16(A + gm * lda + kb) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
            const int c = tid + i * Cfg::kThreads;
            const int row = c / CPR_B, col = c % CPR_B;
            const int64_t kb = (int64_t)kt * RB + col * 16;
            const int gn = n0 + row;
            rb[i] = (gn < N && kb < ldb) ? load16(B + gn * ldb + kb) : i32x4{0, 0, 0, 0};
        }
    };
    auto store_step = [&](int buf) {
        uint8_t *sa = smem + buf * Cfg::STAGE_BYTES;
        uint8_t *sb = sa + Cfg::BM * RA;
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
            const int c = tid + i * Cfg::kThreads;
            *reinterpret_cast<i32x4 *>(sa + swz_offset<CPR_A>(c / CPR_A, c % CPR_A)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
            const int c = tid + i * Cfg::kThreads;
            *reinterpret_cast<i32x4 *>(sb + swz_offset<CPR_B>(c / CPR_B, c % CPR_B)) = rb[i];
        }
    };

    i32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = i32x16{};

    const int h = lane >> 5;     // which 16-k half of an MFMA operand this lane feeds
    const int r32 = lane & 31;   // operand row inside a 32-row block

    if (ktiles > 0) {
        load_step(0);
        store_step(0);
    }
    __syncthreads();

    for (int kt = 0; kt < ktiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ktiles) load_step(kt + 1);

        const uint8_t *sa = smem + buf * Cfg::STAGE_BYTES;
        const uint8_t *sb = sa + Cfg::BM * RA;
#pragma unroll
        for (int p = 0; p < BK / 64; ++p) {
            i32x4 b_lo[FN], b_hi[FN], a_lo[FM], a_hi[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = (wn * FN + fn) * 32 + r32;
                const i32x4 q = *reinterpret_cast<const i32x4 *>(sb + swz_offset<CPR_B>(row, 2 * p + h));
                unpack_chunk<VAR == W4A8>(q, b_lo[fn], b_hi[fn]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = (wm * FM + fm) * 32 + r32;
                if (VAR == I4I4) {
                    const i32x4 q = *reinterpret_cast<const i32x4 *>(sa + swz_offset<CPR_A>(row, 2 * p + h));
                    unpack_chunk<false>(q, a_lo[fm], a_hi[fm]);
                } else {
                    a_lo[fm] = *reinterpret_cast<const i32x4 *>(sa + swz_offset<CPR_A>(row, 4 * p + 2 * h));
                    a_hi[fm] = *reinterpret_cast<const i32x4 *>(sa + swz_offset<CPR_A>(row, 4 * p + 2 * h + 1));
                }
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    acc[fn][fm] = mfma_32x32x32(b_lo[fn], a_lo[fm], acc[fn][fm]);
                    acc[fn][fm] = mfma_32x32x32(b_hi[fn], a_hi[fm], acc[fn][fm]);
                }
        }

        if (kt + 1 < ktiles) store_step(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = l%32 of each column block.
    const bool vec_ok = (N % 4) == 0;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + (wm * FM + fm) * 32 + r32;
            if (m >= M) continue;
            int32_t *crow = C + (int64_t)m * N;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = n0 + (wn * FN + fn) * 32 + 8 * rg + 4 * h;
                const i32x4 v = i32x4{acc[fn][fm][4 * rg + 0], acc[fn][fm][4 * rg + 1],
                                      acc[fn][fm][4 * rg + 2], acc[fn][fm][4 * rg + 3]} >>
                                Cfg::SHIFT;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<i32x4 *>(crow + n) = v;
                } else {
                    if (n + 0 < N) crow[n + 0] = v.x;
                    if (n + 1 < N) crow[n + 1] = v.y;
                    if (n + 2 < N) crow[n + 2] = v.z;
                    if (n + 3 < N) crow[n + 3] = v.w;
                }
            }
        }
}

}  // namespace lpgemm
