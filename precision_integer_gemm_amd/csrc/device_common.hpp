// device_common.hpp -- register-level building blocks shared by the gfx950
// GEMM kernels: int8 MFMA wrappers and the 4-bit -> int8 unpack.
//
// Unpack.  A packed byte holds logical element 2j in its low nibble and 2j+1
// in its high nibble, each a two's-complement 4-bit value (the tutorial's
// pack_int4; the w4a8 PR's torch_convert).  Instead of sign-extending each
// nibble (the w4a8 PR's _tir_u8_to_i4_to_i8 shifts the field to the top of an
// int8 and back), the kernels keep every nibble in the TOP half of its byte:
//     byte & 0xF0         == 16 * (high nibble as signed int4)   (as an int8)
//     (byte << 4) & 0xF0  == 16 * (low nibble as signed int4)
// so a packed dword becomes two dwords of int8 operands in three or five VALU
// operations, and every product carries an exact factor 16 (one 4-bit
// operand) or 256 (two), removed by an arithmetic right shift in the
// epilogue.  Each term is then at most 128*128 = 16384 in magnitude, so the
// int32 accumulator is exact for K <= 131070.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lpgemm {

// Operand formats: int4 x int4, int8 A with packed int4 B, and the fp8 GEMM
// (the second workload: fp32 accumulation) with e4m3 (FP8) or e5m2 (BF8) A
// and B.
enum Variant { I4I4 = 0, W4A8 = 1, FP8 = 2, BF8 = 3 };

// One byte per element on both operands, floating point.
constexpr bool is_fp8(int var) { return var == FP8 || var == BF8; }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// D(32x32) += S0(32x32 rows, 32 k) * S1(32 k, 32 cols); S0 lane l: row l%32,
// S1 lane l: column l%32, both the same 16 k chosen by l/32.  D lane l,
// register r: row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ i32x16 mfma_32x32x32(i32x4 s0, i32x4 s1, i32x16 acc)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(s0, s1, acc, 0, 0, 0);
}

// D(16x16) += S0(16 rows, 64 k) * S1(64 k, 16 cols); S0 lane l: row l%16,
// S1 lane l: column l%16, both the same 16 k chosen by l/16.  D lane l,
// register r: row 4*(l/16) + r, column l%16.
__device__ __forceinline__ i32x4 mfma_16x16x64(i32x4 s0, i32x4 s1, i32x4 acc)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(s0, s1, acc, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// D(32x32, fp32) += S0(32 rows, 64 k) * S1(64 k, 32 cols), both operands fp8
// (FMT 0: e4m3, 1: e5m2, the f8f6f4 MFMA's operand format codes): S0 lane l:
// row l%32, S1 lane l: column l%32, each the 32 consecutive k from 32 (l / 32),
// as two 16-byte halves (lo: the first 16 k).  Products are exact in fp32; the
// sums are not IEEE binary32 (see the fp8 entry points' accuracy contract).
// D layout as mfma_32x32x32.
template <int FMT>
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(i32x4 s0_lo, i32x4 s0_hi, i32x4 s1_lo,
                                                    i32x4 s1_hi, f32x16 acc)
{
    const i32x8 s0 = {s0_lo.x, s0_lo.y, s0_lo.z, s0_lo.w, s0_hi.x, s0_hi.y, s0_hi.z, s0_hi.w};
    const i32x8 s1 = {s1_lo.x, s1_lo.y, s1_lo.z, s1_lo.w, s1_hi.x, s1_hi.y, s1_hi.z, s1_hi.w};
    // scales 2^0 (E8M0 exponent 127) on both operands
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(s0, s1, acc, FMT, FMT, 0, 127, 0, 127);
}

// Split order: 8 nibbles of `d` -> the 4 even-k values (x16) then the 4 odd-k
// values (x16).  Used where both MFMA operands are 4-bit and so share the
// same permutation of k, which leaves every dot product unchanged.
__device__ __forceinline__ void unpack_x16_split(uint32_t d, uint32_t &even, uint32_t &odd)
{
    even = (d << 4) & 0xF0F0F0F0u;
    odd = d & 0xF0F0F0F0u;
}

// Natural order: 8 nibbles of `d` (k0..k7) -> dword [k0 k1 k2 k3] and dword
// [k4 k5 k6 k7], each value x16, matching an int8 operand read in k order.
// v_perm_b32 picks bytes from the pair {hi: d, lo: d << 4}; selector values
// 0-3 name bytes of the low dword, 4-7 bytes of the high dword.
__device__ __forceinline__ void unpack_x16_natural(uint32_t d, uint32_t &k0123, uint32_t &k4567)
{
    const uint32_t y = d << 4;
    k0123 = __builtin_amdgcn_perm(d, y, 0x05010400u) & 0xF0F0F0F0u;
    k4567 = __builtin_amdgcn_perm(d, y, 0x07030602u) & 0xF0F0F0F0u;
}

// 16 packed bytes (32 logical k) -> two MFMA operands of 16 k each.
template <bool NATURAL>
__device__ __forceinline__ void unpack_chunk(const i32x4 q, i32x4 &lo16, i32x4 &hi16)
{
    uint32_t a, b, c, d, e, f, g, h;
    if (NATURAL) {
        unpack_x16_natural((uint32_t)q.x, a, b);
        unpack_x16_natural((uint32_t)q.y, c, d);
        unpack_x16_natural((uint32_t)q.z, e, f);
        unpack_x16_natural((uint32_t)q.w, g, h);
    } else {
        unpack_x16_split((uint32_t)q.x, a, b);
        unpack_x16_split((uint32_t)q.y, c, d);
        unpack_x16_split((uint32_t)q.z, e, f);
        unpack_x16_split((uint32_t)q.w, g, h);
    }
    lo16 = i32x4{(int32_t)a, (int32_t)b, (int32_t)c, (int32_t)d};
    hi16 = i32x4{(int32_t)e, (int32_t)f, (int32_t)g, (int32_t)h};
}

// Sign-extended value of nibble `pos` (0 low, 1 high) of `byte`.
__device__ __forceinline__ int32_t int4_at(uint32_t byte, uint32_t pos)
{
    return ((int32_t)(byte << (28 - 4 * pos))) >> 28;
}

__device__ __forceinline__ i32x4 load16(const void *p)
{
    return *reinterpret_cast<const i32x4 *>(p);
}

// Workgroup barrier for LDS traffic only: drains this wave's LDS operations
// and waits for the other waves, without the vector-memory drain that a full
// __syncthreads() fence adds (prefetched global loads stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer resource over `bytes` bytes at `base`: loads at offsets at or
// past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, offset, 0, 0);
}

// ---- output epilogue -------------------------------------------------------
// The integer result C[m][n] is stored either as int32, or scaled per row and
// per column and converted (the one-K-block case of the tutorial's
// gemm_blockscaled, with fp32 arithmetic):
//     D[m][n] = out(((float)C[m][n] * scale_a[m]) * scale_b[n])
// where (float) and both multiplies round to nearest even in fp32 and out()
// converts to fp32 (identity), bf16 or fp16, rounding to nearest even.
enum OutFormat { OUT_I32 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_F16 = 3, OUT_E4M3 = 4, OUT_E5M2 = 5 };

struct Epilogue {
    void *out;             // D (or C), row-major [M][N]
    const float *scale_a;  // [M], scaled formats only; SFA [M][nb] with block scales
    const float *scale_b;  // [N], scaled formats only; SFB [N][nb] with block scales
    int32_t nb = 0;        // block scales: number of K blocks, ceil(K / g)
    int32_t lg = 0;        // block scales: log2 of the block length g
};

// fp32 -> bf16 bits, round to nearest even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f16_bits_rne(float x)
{
    const _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float scaled(int32_t c, float sa, float sb)
{
    const float t = (float)c;
    const float y = t * sa;
    float z = y * sb;
    // Materialise the binary32 product: without this the compiler folds the
    // last multiply and a following fp16 conversion into one fused operation
    // (one rounding instead of two, and -0 turned into +0).
    asm volatile("" : "+v"(z));
    return z;
}

template <int OUT>
__device__ __forceinline__ uint32_t out_bits(float y)
{
    if (OUT == OUT_BF16) return bf16_bits_rne(y);
    return f16_bits_rne(y);
}

// Store results v[i] for columns n .. n+3 of row m (columns >= N skipped).
// sa is scale_a[m]; sb[i] scale_b[n + i] (read only for columns < N).  The
// 16-byte (int32 / fp32) or 8-byte (bf16 / fp16) vector store is used when
// all four columns exist and N % 4 == 0 (aligned base assumed).
template <int OUT>
__device__ __forceinline__ void store_row4(const Epilogue &e, int64_t m, int N, int n, i32x4 v,
                                           float sa, const float (&sb)[4])
{
    const bool vec = (N % 4) == 0 && n + 3 < N;
    if (OUT == OUT_I32) {
        int32_t *row = static_cast<int32_t *>(e.out) + m * N;
        if (vec) {
            *reinterpret_cast<i32x4 *>(row + n) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = v[i];
        }
    } else if (OUT == OUT_F32) {
        float *row = static_cast<float *>(e.out) + m * N;
        if (vec) {
            i32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (int32_t)__float_as_uint(scaled(v[i], sa, sb[i]));
            *reinterpret_cast<i32x4 *>(row + n) = w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = scaled(v[i], sa, sb[i]);
        }
    } else {
        uint16_t *row = static_cast<uint16_t *>(e.out) + m * N;
        if (vec) {
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = out_bits<OUT>(scaled(v[i], sa, sb[i]));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2 *>(row + n) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = (uint16_t)out_bits<OUT>(scaled(v[i], sa, sb[i]));
        }
    }
}

// C[m][n + i] += v[i] for the columns that exist (int32 atomics, no return):
// partial sums of K ranges, added into a C zeroed beforehand.
__device__ __forceinline__ void atomic_add_row4(const Epilogue &e, int64_t m, int N, int n, i32x4 v)
{
    int32_t *row = static_cast<int32_t *>(e.out) + m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (n + i < N) __hip_atomic_fetch_add(row + n + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// scale_a[m] (scaled formats; 0 otherwise).
template <int OUT>
__device__ __forceinline__ float load_scale_a(const Epilogue &e, int64_t m)
{
    return OUT == OUT_I32 ? 0.f : e.scale_a[m];
}

// scale_b[n .. n+3], zero where the column does not exist: one 16-byte load
// when the four columns exist and the address is 16-byte aligned.
template <int OUT>
__device__ __forceinline__ void load_scale_b4(const Epilogue &e, int N, int n, float (&sb)[4])
{
    if (OUT == OUT_I32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[i] = 0.f;
        return;
    }
    const float *p = e.scale_b + n;
    if (n + 3 < N && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        sb[0] = v.x;
        sb[1] = v.y;
        sb[2] = v.z;
        sb[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[i] = (n + i < N) ? p[i] : 0.f;
    }
}

// Both scale sets of one row segment.
template <int OUT>
__device__ __forceinline__ void load_scales(const Epilogue &e, int64_t m, int N, int n, float &sa,
                                            float (&sb)[4])
{
    sa = load_scale_a<OUT>(e, m);
    load_scale_b4<OUT>(e, N, n, sb);
}

// ---- fp8 (e4m3) values -----------------------------------------------------
// E4M3 as in the OCP 8-bit formats: bit 7 sign, bits 6..3 exponent (bias 7),
// bits 2..0 mantissa; exponent 0 subnormal (m * 2^-9); S.1111.111 NaN; no
// infinities; largest finite 448.

// Value of code c.
__device__ __forceinline__ float e4m3_to_float(uint32_t c)
{
    const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
    if (e == 15u && m == 7u) return __uint_as_float(s | 0x7FC00000u);
    if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));  // m * 2^-9
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// Nearest code of x, ties to even, magnitudes of 448 and above saturating to
// +-448; NaN gives the NaN code (with x's sign).
__device__ __forceinline__ uint32_t float_to_e4m3(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t s = (u >> 24) & 0x80u, ax = u & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return s | 0x7Fu;
    if (ax >= 0x43E00000u) return s | 0x7Eu;  // 448 and beyond (inf included)
    if (ax >= 0x3C800000u) {                    // normal: |x| >= 2^-6
        // keep 3 mantissa bits, nearest-even on the 20 dropped ones; a carry
        // moves into the exponent as it should
        const uint32_t r = (ax + 0x7FFFFu + ((ax >> 20) & 1u)) >> 20;
        return s | (r - (120u << 3));
    }
    // subnormal: quantum 2^-9; the product is exact, rint rounds to even
    return s | (uint32_t)__builtin_rintf(__uint_as_float(ax) * 512.0f);
}

// ---- fp8 (e5m2) values -----------------------------------------------------
// E5M2 as in the OCP 8-bit formats (the top byte of an IEEE binary16): bit 7
// sign, bits 6..2 exponent (bias 15), bits 1..0 mantissa; exponent 0
// subnormal (m * 2^-16); exponent 31 infinity (m = 0) or NaN; largest finite
// 57344.

// Value of code c.
__device__ __forceinline__ float e5m2_to_float(uint32_t c)
{
    const uint32_t s = (c & 0x80u) << 24, e = (c >> 2) & 31u, m = c & 3u;
    if (e == 31u) return __uint_as_float(s | (m ? 0x7FC00000u : 0x7F800000u));
    if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 1.52587890625e-05f));  // m * 2^-16
    return __uint_as_float(s | ((e + 112u) << 23) | (m << 21));
}

// Nearest code of x, ties to even; magnitudes from 61440 (the midpoint above
// the largest finite value, which ties to the even neighbour 2^16) become
// infinity; NaN gives a NaN code with x's sign.
__device__ __forceinline__ uint32_t float_to_e5m2(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t s = (u >> 24) & 0x80u, ax = u & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return s | 0x7Fu;
    if (ax >= 0x47700000u) return s | 0x7Cu;  // 61440 and beyond (inf included)
    if (ax >= 0x38800000u) {                    // normal: |x| >= 2^-14
        // keep 2 mantissa bits, nearest-even on the 21 dropped ones
        const uint32_t r = (ax + 0xFFFFFu + ((ax >> 21) & 1u)) >> 21;
        return s | (r - (112u << 2));
    }
    // subnormal: quantum 2^-16; the product is exact, rint rounds to even
    return s | (uint32_t)__builtin_rintf(__uint_as_float(ax) * 65536.0f);
}

// Store fp32 results v[i] for columns n .. n+3 of row m (columns >= N
// skipped) as fp32, bf16, fp16, e4m3 or e5m2 (nearest even).  Vector stores
// when all four exist and N % 4 == 0.
template <int OUT>
__device__ __forceinline__ void store_row4f(const Epilogue &e, int64_t m, int N, int n, const float (&v)[4])
{
    const bool vec = (N % 4) == 0 && n + 3 < N;
    if (OUT == OUT_BF16 || OUT == OUT_F16) {
        uint16_t *row = static_cast<uint16_t *>(e.out) + m * N;
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = v[i];
            asm volatile("" : "+v"(x));  // convert the binary32 value itself (no fused rounding)
            hb[i] = out_bits<OUT>(x);
        }
        if (vec) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2 *>(row + n) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = (uint16_t)hb[i];
        }
    } else if (OUT == OUT_F32) {
        float *row = static_cast<float *>(e.out) + m * N;
        if (vec) {
            *reinterpret_cast<i32x4 *>(row + n) =
                i32x4{(int32_t)__float_as_uint(v[0]), (int32_t)__float_as_uint(v[1]),
                      (int32_t)__float_as_uint(v[2]), (int32_t)__float_as_uint(v[3])};
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = v[i];
        }
    } else {
        uint8_t *row = static_cast<uint8_t *>(e.out) + m * N;
        auto enc = [](float f) { return OUT == OUT_E5M2 ? float_to_e5m2(f) : float_to_e4m3(f); };
        if (vec) {
            *reinterpret_cast<uint32_t *>(row + n) = enc(v[0]) | (enc(v[1]) << 8) | (enc(v[2]) << 16) |
                                                      (enc(v[3]) << 24);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) row[n + i] = (uint8_t)enc(v[i]);
        }
    }
}

// ---- direct-to-LDS loads ---------------------------------------------------
// Buffer resource for `bytes` bytes at `base` (raw buffer, no stride).
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)p);
    r.y = __builtin_amdgcn_readfirstlane((int32_t)((p >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r.w = 0x00020000;  // 32-bit data format: raw byte-addressed loads
    return r;
}

// 16 bytes per lane from rsrc[voffset] into LDS at lds_base + 16 * lane.  An
// offset at or beyond the resource size reads zeros.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voffset, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"  // one wait state between an M0 write and an LDS DMA
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voffset), "s"(rsrc), "s"(lds_base)
        : "memory");
}

// 4 bytes per lane from rsrc[voffset] into LDS at lds_base + 4 * lane (the
// per-K-block scale tables, one float per lane from anywhere in the table).
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voffset, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voffset), "s"(rsrc), "s"(lds_base)
        : "memory");
}

// dma16 with the non-temporal hint, for data that is read exactly once (the
// narrow-M kernel's weight stream).  Measured on MI355X: right after a kernel
// that wrote 268 MB, a 117 MB weight stream read this way ran in half the time
// that plain loads took there; on an idle memory system both run alike.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voffset, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voffset), "s"(rsrc), "s"(lds_base)
        : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (the counter holds 0..63; a larger N waits for 63, which is only stricter).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N < 63 ? N : 63) : "memory");
}

// A buffer offset that no resource here reaches: such a load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

}  // namespace lpgemm
