// gemm_general.hpp -- kernels for shapes and layouts the fast paths do not
// take (K not a multiple of 32, unaligned bases), the K == 0 fill, and the
// device pack / unpack of 4-bit operands.
#pragma once

#include "device_common.hpp"

namespace lpgemm {

// One thread per output element, bytes read one at a time: correct for any
// even K and any alignment.  Sums fit int32 exactly (|C| <= 1024*K).  Also
// serves K == 0 for the scaled formats (the empty sum, then scaled).
template <int VAR, int OUT>
__global__ __launch_bounds__(256) void gemm_general_kernel(const uint8_t *__restrict__ A,
                                                           const uint8_t *__restrict__ B,
                                                           Epilogue epi, int64_t M, int64_t N,
                                                           int64_t K)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
    if (m >= M || n >= N) return;
    const int64_t half = K / 2;
    const uint8_t *brow = B + n * half;
    int32_t sum = 0;
    if (VAR == I4I4) {
        const uint8_t *arow = A + m * half;
        for (int64_t j = 0; j < half; ++j) {
            const uint32_t a = arow[j], b = brow[j];
            sum += int4_at(a, 0) * int4_at(b, 0) + int4_at(a, 1) * int4_at(b, 1);
        }
    } else {
        const int8_t *arow = reinterpret_cast<const int8_t *>(A) + m * K;
        for (int64_t j = 0; j < half; ++j) {
            const uint32_t b = brow[j];
            sum += (int32_t)arow[2 * j] * int4_at(b, 0) + (int32_t)arow[2 * j + 1] * int4_at(b, 1);
        }
    }
    if (OUT == OUT_I32) {
        static_cast<int32_t *>(epi.out)[m * N + n] = sum;
    } else {
        const float y = scaled(sum, epi.scale_a[m], epi.scale_b[n]);
        if (OUT == OUT_F32)
            static_cast<float *>(epi.out)[m * N + n] = y;
        else
            static_cast<uint16_t *>(epi.out)[m * N + n] = (uint16_t)out_bits<OUT>(y);
    }
}

// Per-K-block scaled product, one thread per output element: block j (k in
// [j g, min(K, (j+1) g)), g = 2^epi.lg, epi.nb blocks) is summed exactly in
// int32, then ((float)C_j * SFA[m][j]) * SFB[n][j] is added to a binary32
// accumulator in increasing j, every step rounding to nearest even; the
// accumulator starts at -0 (so the first term is taken as it is), or is +0
// when there is no block (K == 0).  Any even K and any alignment.
template <int VAR, int OUT>
__global__ __launch_bounds__(256) void gemm_blockscaled_general_kernel(const uint8_t *__restrict__ A,
                                                                       const uint8_t *__restrict__ B,
                                                                       Epilogue epi, int64_t M,
                                                                       int64_t N, int64_t K)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
    if (m >= M || n >= N) return;
    const int64_t half = K / 2, g2 = ((int64_t)1 << epi.lg) / 2, nb = epi.nb;
    const uint8_t *brow = B + n * half;
    const float *sfa = epi.scale_a + m * nb, *sfb = epi.scale_b + n * nb;
    float acc = nb > 0 ? -0.0f : 0.0f;
    for (int64_t j = 0; j < nb; ++j) {
        const int64_t p0 = j * g2, p1 = min(half, p0 + g2);  // byte pairs of the block
        int32_t c = 0;
        if (VAR == I4I4) {
            const uint8_t *arow = A + m * half;
            for (int64_t q = p0; q < p1; ++q) {
                const uint32_t a = arow[q], b = brow[q];
                c += int4_at(a, 0) * int4_at(b, 0) + int4_at(a, 1) * int4_at(b, 1);
            }
        } else {
            const int8_t *arow = reinterpret_cast<const int8_t *>(A) + m * K;
            for (int64_t q = p0; q < p1; ++q) {
                const uint32_t b = brow[q];
                c += (int32_t)arow[2 * q] * int4_at(b, 0) + (int32_t)arow[2 * q + 1] * int4_at(b, 1);
            }
        }
        acc = acc + scaled(c, sfa[j], sfb[j]);
    }
    asm volatile("" : "+v"(acc));  // convert the binary32 value itself
    if (OUT == OUT_F32)
        static_cast<float *>(epi.out)[m * N + n] = acc;
    else
        static_cast<uint16_t *>(epi.out)[m * N + n] = (uint16_t)out_bits<OUT>(acc);
}

// fp8 product (VAR: FP8 e4m3 or BF8 e5m2 operands), one thread per output:
// exact products summed in fp32 in k order; fp32 output, or the operands' fp8
// format (OUT_E4M3 / OUT_E5M2).  Any K and alignment.
template <int VAR, int OUT>
__global__ __launch_bounds__(256) void gemm_fp8_general_kernel(const uint8_t *__restrict__ A,
                                                               const uint8_t *__restrict__ B,
                                                               Epilogue epi, int64_t M, int64_t N,
                                                               int64_t K)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
    if (m >= M || n >= N) return;
    const uint8_t *arow = A + m * K, *brow = B + n * K;
    auto dec = [](uint32_t c) { return VAR == BF8 ? e5m2_to_float(c) : e4m3_to_float(c); };
    float sum = 0.f;
    for (int64_t k = 0; k < K; ++k) {
        const float p = dec(arow[k]) * dec(brow[k]);  // exact
        sum += p;
    }
    if (OUT == OUT_F32)
        static_cast<float *>(epi.out)[m * N + n] = sum;
    else
        static_cast<uint8_t *>(epi.out)[m * N + n] =
            (uint8_t)(OUT == OUT_E5M2 ? float_to_e5m2(sum) : float_to_e4m3(sum));
}

// C[0 .. count) = 0: the empty sum (K == 0).  A kernel, not a memset, so the
// call stays capturable in a graph.
__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t *__restrict__ C, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        C[i] = 0;
}

// C[i] = sum over c < slices of W[c * count + i]: the partial sums of K ranges
// (exact in int32, any order).  Four elements per thread when count % 4 == 0
// (16-byte aligned W and C), else one.
__global__ __launch_bounds__(256) void sum_slices_kernel(const int32_t *__restrict__ W,
                                                         int32_t *__restrict__ C, int64_t count,
                                                         int slices)
{
    typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (count % 4 == 0) {
        const i32x4v *w = reinterpret_cast<const i32x4v *>(W);
        i32x4v *c4 = reinterpret_cast<i32x4v *>(C);
        const int64_t n4 = count / 4;
        for (int64_t i = t; i < n4; i += stride) {
            i32x4v s = w[i];
            for (int k = 1; k < slices; ++k) s += w[(int64_t)k * n4 + i];
            c4[i] = s;
        }
    } else {
        for (int64_t i = t; i < count; i += stride) {
            int32_t s = W[i];
            for (int k = 1; k < slices; ++k) s += W[(int64_t)k * count + i];
            C[i] = s;
        }
    }
}

// packed[r][j] = (x[r][2j] & 0xF) | ((x[r][2j+1] & 0xF) << 4), one thread per
// output byte (grid-stride over rows * K/2).
__global__ __launch_bounds__(256) void pack_int4_kernel(const int8_t *__restrict__ logical,
                                                        uint8_t *__restrict__ packed,
                                                        int64_t total_bytes)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_bytes; i += stride) {
        const uint32_t even = (uint32_t)(uint8_t)logical[2 * i] & 0xFu;
        const uint32_t odd = (uint32_t)(uint8_t)logical[2 * i + 1] & 0xFu;
        packed[i] = (uint8_t)(even | (odd << 4));
    }
}

// logical[r][2j + p] = sign-extended nibble p of packed[r][j].
__global__ __launch_bounds__(256) void unpack_int4_kernel(const uint8_t *__restrict__ packed,
                                                          int8_t *__restrict__ logical,
                                                          int64_t total_bytes)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_bytes; i += stride) {
        const uint32_t b = packed[i];
        logical[2 * i] = (int8_t)int4_at(b, 0);
        logical[2 * i + 1] = (int8_t)int4_at(b, 1);
    }
}

}  // namespace lpgemm
