// gemm_skinny.hpp -- narrow-M W4A8 kernel for gfx950 (decode-like shapes).
//
// For M <= 16 the product is bound by reading the packed weights B once from
// HBM.  Design:
//   * workgroup = KW waves; wave w owns the w-th slice of K (KSTEPS steps of
//     128 logical k) for the whole kernel and keeps the matching fragments of
//     A (rows zero-padded to 16) in registers, loaded once;
//   * the workgroup walks strips of 16 rows of B (grid-stride); for each strip
//     a wave issues all KSTEPS of its 16-byte-per-lane loads at once, two
//     strips ahead of the strip it computes (three register sets used in
//     turn: no copy ever waits on a prefetch), so about 128 KB per compute
//     unit stay in flight;
//   * loads are raw buffer loads: rows past N come back as zeros from the
//     range check, steps past K use an out-of-range offset -- no branches;
//   * nibbles are unpacked in registers and contracted with
//     v_mfma_i32_16x16x64_i8, B as the MFMA's 16-row operand and A as its
//     16-column operand (the w4a8 page's kernel also puts the dequantised B
//     first and produces C^T), so each lane ends with four consecutive n of
//     one m;
//   * the KW partial tiles are summed in LDS in a fixed order (exact; no
//     atomics, no memset) and wave 0 stores the strip of C.
//
// Requirements (checked on the host): M <= 16, K % 32 == 0, 16-byte aligned
// bases, N * K / 2 < 2^31, KW * KSTEPS * 128 >= K, at most 256 workgroups
// (so offsets of the strips prefetched past the end still fit 32 bits).
#pragma once

#include "device_common.hpp"

namespace lpgemm {

template <int KW, int KSTEPS>
__global__ __launch_bounds__(64 * KW) void gemm_w4a8_skinny_kernel(
    const int8_t *__restrict__ A, const uint8_t *__restrict__ B, int32_t *__restrict__ C, int M,
    int N, int K)
{
    constexpr uint32_t kOut = 0x80000000u;  // an offset no resource here reaches
    __shared__ i32x4 red[2][KW][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;    // k group this lane feeds
    const int r16 = lane & 15;  // operand row (n for B, m for A)
    const int strips = (N + 15) / 16;
    const uint32_t ldb = (uint32_t)K / 2;
    const int k_begin = wave * (KSTEPS * 128);

    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(A, (uint32_t)M * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(B, (uint32_t)N * ldb);

    // A fragments of this wave's K slice: step j covers logical k
    // k_begin + 128 j + [32 g, 32 g + 32) of row r16, as two 16-byte halves.
    // Rows past M lie past the resource and read as zeros.
    i32x4 a_lo[KSTEPS], a_hi[KSTEPS];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
        const int kl = k_begin + 128 * j + 32 * g;
        const uint32_t off = kl < K ? (uint32_t)r16 * (uint32_t)K + (uint32_t)kl : kOut;
        a_lo[j] = buffer_load16(rsrc_a, off);
        a_hi[j] = buffer_load16(rsrc_a, off == kOut ? kOut : off + 16);
    }

    // Packed B of strip s for every step of this wave's slice (16 bytes per
    // lane per step: logical k k_begin + 128 j + [32 g, 32 g + 32) of row n).
    auto load_strip = [&](int s, i32x4(&q)[KSTEPS]) {
        const uint32_t row_off = (uint32_t)(s * 16 + r16) * ldb;
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
            const int kl = k_begin + 128 * j + 32 * g;
            q[j] = buffer_load16(rsrc_b, kl < K ? row_off + (uint32_t)kl / 2 : kOut);
        }
    };

    int buf = 0;
    auto do_strip = [&](int s, const i32x4(&q)[KSTEPS]) {
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
            i32x4 b_lo, b_hi;
            unpack_chunk<true>(q[j], b_lo, b_hi);
            acc = mfma_16x16x64(b_lo, a_lo[j], acc);
            acc = mfma_16x16x64(b_hi, a_hi[j], acc);
        }
        red[buf][wave][lane] = acc;
        lds_barrier();
        if (wave == 0) {
            i32x4 sum = red[buf][0][lane];
#pragma unroll
            for (int w = 1; w < KW; ++w) sum += red[buf][w][lane];
            sum >>= 4;  // B carried a factor 16
            const int m = r16;
            const int n = s * 16 + 4 * g;
            if (m < M) {
                int32_t *crow = C + (int64_t)m * N;
                if ((N % 4) == 0 && n + 3 < N) {
                    *reinterpret_cast<i32x4 *>(crow + n) = sum;
                } else {
                    if (n + 0 < N) crow[n + 0] = sum.x;
                    if (n + 1 < N) crow[n + 1] = sum.y;
                    if (n + 2 < N) crow[n + 2] = sum.z;
                    if (n + 3 < N) crow[n + 3] = sum.w;
                }
            }
        }
        // The next strip writes the other half of `red`, so one barrier per
        // strip suffices: wave 0 has finished reading this half before any
        // wave passes the next strip's barrier.
        buf ^= 1;
    };

    // Strips are prefetched two ahead into three register sets used in turn.
    // The prefetch is unconditional: a strip past the end reads zeros (its
    // offsets lie past the resource), which keeps the number of loads in
    // flight fixed so the compiler waits only for the strip being computed.
    const int G = gridDim.x;
    int s = blockIdx.x;
    i32x4 q0[KSTEPS], q1[KSTEPS], q2[KSTEPS];
    load_strip(s, q0);
    load_strip(s + G, q1);
    while (s < strips) {
        load_strip(s + 2 * G, q2);
        do_strip(s, q0);
        s += G;
        if (s >= strips) break;
        load_strip(s + 2 * G, q0);
        do_strip(s, q1);
        s += G;
        if (s >= strips) break;
        load_strip(s + 2 * G, q1);
        do_strip(s, q2);
        s += G;
    }
}

}  // namespace lpgemm
