// ceiling_probe.hip -- what the matrix cores and the LDS sustain, measured.
//
// Measurement support beside the GEMM library (its own shared object,
// _ceiling.so, loaded only by bench.py): each kernel keeps one unit of a
// compute unit busy for a fixed number of iterations, so that a caller can
// time it and set a GEMM's throughput against what the chip sustains under
// that load, clock reduction included, next to the published peak.
//
// Every kernel requests 96 KB of (unused) dynamic LDS, so a compute unit holds
// exactly one workgroup, and the grid is one workgroup per compute unit.
//
//   kind 0  FP6 (E3M2) v_mfma_scale_f32_32x32x64_f8f6f4, 4 waves (one per
//           SIMD), 8 independent accumulators each: matrix cores only.
//   kind 1  int8 v_mfma_i32_32x32x32_i8, same structure.
//   kind 2  fp8 (E4M3) v_mfma_scale_f32_32x32x64_f8f6f4, same structure.
//   kind 3  LDS reads only: 8 waves, ds_read_b128 + ds_read_b64 of
//           lane-linear 1.5 KB fragments, folded into a register.
//   kind 4  the FP6 GEMM's inner loop without global memory: 8 waves (two
//           per SIMD) of 4 x 2 blocks of 32 x 32, per 64 k six 1.5 KB
//           fragments read from LDS one step ahead and eight MFMAs.
//
// Work per launch (ceiling_probe_work): kinds 0-2 and 4 in operations
// (2 x MACs), kind 3 in LDS bytes read.
//
// Kinds 0-2 and 4 also report the shader clock they ran at: thread 0 of each
// workgroup reads the shader-clock counter (s_memtime) and the constant-rate
// counter (s_memrealtime) before and after its loop.
//
// ceiling_probe_stream_sweep is the HBM counterpart: one pass over a caller's
// buffer, every byte read once (what a single streaming pass of that size
// reaches, launch and ramp included, for the memory-bound GEMM shapes), in one
// configuration of a family: buffer loads with a chosen cache policy and
// loads in flight per thread, or direct-to-LDS loads of 1 KB per wave
// instruction (the narrow-M GEMM's way of streaming its weights), with a
// chosen number of workgroups.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"

namespace {

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLdsRequest = 96 * 1024;
constexpr int kFrag = 1536;
constexpr int kChains = 8;

// Operand registers: arbitrary nonzero bit patterns that differ per lane
// (finite in every format used here: E3M2 has no specials, and the E4M3 mask
// clears the lowest exponent bit so no code is a NaN).
__device__ inline i32x8 operand(uint32_t seed, uint32_t mask)
{
    i32x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (int32_t)(((seed + 0x9E3779B9u * (i + 1)) * 2654435761u) & mask);
    return v;
}

// Shader-clock and constant-rate counters at the start of a probe loop.
struct Clocks {
    uint64_t shader, real;
};

__device__ inline Clocks clocks_now()
{
    return Clocks{__builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime()};
}

// Thread 0 writes its workgroup's shader-clock and constant-rate ticks.
__device__ inline void clocks_store(int64_t *clk, const Clocks &t0)
{
    if (clk != nullptr && threadIdx.x == 0) {
        const Clocks t1 = clocks_now();
        clk[2 * blockIdx.x] = (int64_t)(t1.shader - t0.shader);
        clk[2 * blockIdx.x + 1] = (int64_t)(t1.real - t0.real);
    }
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float *out, int iters, int64_t *clk)
{
    const Clocks t0 = clocks_now();
    const uint32_t seed = threadIdx.x * 977u + blockIdx.x;
    const uint32_t mask = KIND == 2 ? 0x77777777u : 0xFFFFFFFFu;
    const i32x8 a = operand(seed, mask), b = operand(seed ^ 0x5555u, mask);
    float s = 0.f;
    if constexpr (KIND == 1) {
        const i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
        i32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = i32x16{};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c) s += (float)acc[c][threadIdx.x & 15];
    } else {
        constexpr int fmt = KIND == 0 ? 3 : 0;  // E3M2 or E4M3 operands
        f32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], fmt, fmt, 0, 127,
                                                                          0, 127);
#pragma unroll
        for (int c = 0; c < kChains; ++c) s += acc[c][threadIdx.x & 15];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    clocks_store(clk, t0);
}

// LDS image shared by kinds 3 and 4: four buffers of six fragments (36 KB),
// rotated per step so no read is loop-invariant.
constexpr int kFrags = 6, kBufs = 4;
constexpr int kImage = kBufs * kFrags * kFrag;

__device__ inline void fill_image(uint8_t *lds)
{
    for (int i = threadIdx.x * 4; i < kImage; i += blockDim.x * 4)
        *reinterpret_cast<uint32_t *>(lds + i) = ((uint32_t)i * 2654435761u) & 0x7DF7DF7Du;
    __syncthreads();
}

__device__ inline i32x8 frag_at(const uint8_t *lds, int buf, int f, int lane)
{
    const uint8_t *p = lds + (buf * kFrags + f) * kFrag;
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(p + 16 * lane);
    const i32x2 hi = *reinterpret_cast<const i32x2 *>(p + 1024 + 8 * lane);
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, 0, 0};
}

__global__ __launch_bounds__(512) void lds_loop(float *out, int iters, int64_t *clk)
{
    const Clocks t0 = clocks_now();
    extern __shared__ __align__(16) uint8_t lds[];
    fill_image(lds);
    const int lane = threadIdx.x & 63;
    i32x8 x = {};
    for (int it = 0; it < iters; ++it) {
        const int buf = it & (kBufs - 1);
#pragma unroll
        for (int f = 0; f < kFrags; ++f) x ^= frag_at(lds, buf, f, lane);
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(x[0] ^ x[3] ^ x[5]);
    clocks_store(clk, t0);
}

__global__ __launch_bounds__(512) void lds_mfma_loop(float *out, int iters, int64_t *clk)
{
    const Clocks t0 = clocks_now();
    constexpr int FM = 4, FN = 2;
    static_assert(FM + FN == kFrags, "one buffer holds one step's fragments");
    extern __shared__ __align__(16) uint8_t lds[];
    fill_image(lds);
    const int lane = threadIdx.x & 63;
    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};
    i32x8 cur[kFrags], nxt[kFrags];
#pragma unroll
    for (int f = 0; f < kFrags; ++f) cur[f] = frag_at(lds, 0, f, lane);
    for (int it = 0; it < iters; ++it) {
        const int buf = (it + 1) & (kBufs - 1);
#pragma unroll
        for (int f = 0; f < kFrags; ++f) nxt[f] = frag_at(lds, buf, f, lane);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    cur[fn], cur[FN + fm], acc[fn][fm], 3, 3, 0, 127, 0, 127);
#pragma unroll
        for (int f = 0; f < kFrags; ++f) cur[f] = nxt[f];
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) s += acc[i][j][lane & 15];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    clocks_store(clk, t0);
}

int threads_of(int kind) { return kind >= 3 ? 512 : 256; }

// Buffer-load pass: thread t folds 16-byte elements t, t + S, ... (S = grid
// threads), F loads issued before any is used, each with cache policy POL
// (the buffer instruction's sc0 / nt / sc1 bits).
template <int F, int POL>
__global__ void stream_buf(const void *base, int bytes, int64_t n, int32_t *out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = lpgemm::buffer_rsrc(base, (uint32_t)bytes);
    int32_t fold = 0;
    for (int64_t base = t; base < n; base += stride * F) {
        i32x4 v[F];
#pragma unroll
        for (int u = 0; u < F; ++u) {
            const int64_t i = base + u * stride;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, i < n ? (uint32_t)(i * 16) : lpgemm::kOutOfRange, 0, POL);
        }
#pragma unroll
        for (int u = 0; u < F; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[t] = fold;
}

// Direct-to-LDS pass: wave w of the grid copies 1 KB pieces w, w + W, ...
// (W = grid waves) into its own F-slot LDS ring, keeping F in flight; the
// data is not read back.  NT: the non-temporal hint of the narrow-M kernel.
template <int F, bool NT>
__global__ void stream_dma(i32x4 rsrc, int64_t pieces, int32_t *out)
{
    extern __shared__ __align__(1024) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const uint32_t ring = (uint32_t)reinterpret_cast<uintptr_t>(lds) + (uint32_t)(wave * F) * 1024u;
    const int64_t total = (int64_t)gridDim.x * waves;
    int slot = 0;
    for (int64_t p = (int64_t)blockIdx.x * waves + wave; p < pieces; p += total) {
        const uint32_t off = (uint32_t)(p * 1024) + 16u * (uint32_t)lane;
        if (NT)
            lpgemm::dma16_nt(rsrc, off, ring + (uint32_t)slot * 1024u);
        else
            lpgemm::dma16(rsrc, off, ring + (uint32_t)slot * 1024u);
        slot = slot + 1 == F ? 0 : slot + 1;
        lpgemm::wait_vmcnt<F - 1>();
    }
    lpgemm::wait_vmcnt<0>();
    if (lane == 0) out[(int64_t)blockIdx.x * waves + wave] = slot;
}

// Direct-to-LDS pass in the narrow-M GEMM's own pattern: the buffer is taken
// as 64 KB strips (16 rows of 4 KB), workgroup b copying strips b, b + G, ...
// (G = grid size) and wave w of its 16 copying row w as four 1 KB `nt`
// pieces.  F = 0: one strip per workgroup in flight -- issue its pieces, wait
// for them, barrier, next strip (the GEMM's schedule without its arithmetic);
// F > 0: F pieces in flight per wave, no barrier.  The data is not read back.
template <int F>
__global__ __launch_bounds__(1024) void stream_strips(i32x4 rsrc, int64_t strips, int32_t *out)
{
    extern __shared__ __align__(1024) uint8_t lds[];
    constexpr int kSlots = F == 0 ? 4 : F;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ring = (uint32_t)reinterpret_cast<uintptr_t>(lds) + (uint32_t)(wave * kSlots) * 1024u;
    int slot = 0;
    for (int64_t s = blockIdx.x; s < strips; s += gridDim.x) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            lpgemm::dma16_nt(rsrc, (uint32_t)(s * 65536) + (uint32_t)(wave * 4096 + t * 1024 + 16 * lane),
                             ring + (uint32_t)slot * 1024u);
            slot = slot + 1 == kSlots ? 0 : slot + 1;
            if constexpr (F > 0) lpgemm::wait_vmcnt<F - 1>();
        }
        if constexpr (F == 0) {
            lpgemm::wait_vmcnt<0>();
            lpgemm::lds_barrier();
        }
    }
    lpgemm::wait_vmcnt<0>();
    if (lane == 0) out[(int64_t)blockIdx.x * 16 + wave] = slot;
}

// C-store patterns: one 256 x 256 int32 tile per 512-thread workgroup of an
// M x N row-major matrix (M, N multiples of 256), tile t at tile row t / (N / 256).
//   P = 0: the tiled GEMMs' MFMA layout: wave w (wm = w / 4, wn = w % 4) holds
//          4 x 2 blocks of 32 x 32; each instruction writes 16 bytes at row
//          (wm 4 + fm) 32 + lane % 32, column (wn 2 + fn) 32 + 8 rg + 4 (lane / 32),
//          i.e. 32 bytes of each of 32 rows;
//   P = 1: whole rows: wave w writes rows w, w + 8, ..., one 1 KB row per instruction;
//   P = 2: P = 0's registers written into LDS in two passes of 128 rows (rows
//          padded by 16 bytes), each followed by P = 1's stores of those rows
//          (the GEMMs' last-tile epilogue).
// Element (m, n .. n + 3) holds {m, n, 0, 0} in every pattern.
template <int P>
__global__ __launch_bounds__(512) void store_pattern(int32_t *C, int N)
{
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int kPitch = 1024 + 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / 4, wn = w % 4, r32 = lane & 31, h = lane >> 5;
    const int tiles_n = N / 256;
    const int tm0 = ((int)blockIdx.x / tiles_n) * 256, tn0 = ((int)blockIdx.x % tiles_n) * 256;
    if constexpr (P == 1) {
        for (int r = w; r < 256; r += 8)
            *reinterpret_cast<i32x4 *>(C + (int64_t)(tm0 + r) * N + tn0 + 4 * lane) = i32x4{tm0 + r, tn0 + 4 * lane, 0, 0};
    } else {
        for (int half = 0; half < (P == 2 ? 2 : 1); ++half) {
            if (P == 2 && half) __syncthreads();
            for (int fn = 0; fn < 2; ++fn)
                for (int fm = 0; fm < 4; ++fm) {
                    const int rt = (wm * 4 + fm) * 32 + r32;  // row in the tile
                    if (P == 2 && rt / 128 != half) continue;
                    for (int rg = 0; rg < 4; ++rg) {
                        const int nt = (wn * 2 + fn) * 32 + 8 * rg + 4 * h;
                        const i32x4 v = i32x4{tm0 + rt, tn0 + nt, 0, 0};
                        if constexpr (P == 0)
                            *reinterpret_cast<i32x4 *>(C + (int64_t)(tm0 + rt) * N + tn0 + nt) = v;
                        else
                            *reinterpret_cast<i32x4 *>(lds + (rt - 128 * half) * kPitch + 4 * nt) = v;
                    }
                }
            if constexpr (P == 2) {
                __syncthreads();
                for (int r = w; r < 128; r += 8)
                    *reinterpret_cast<i32x4 *>(C + (int64_t)(tm0 + 128 * half + r) * N + tn0 + 4 * lane) =
                        *reinterpret_cast<const i32x4 *>(lds + r * kPitch + 16 * lane);
            }
        }
    }
}

}  // namespace

// One launch of C-store pattern `pattern` (0, 1, 2: see store_pattern) over
// the M x N int32 matrix C (device, M and N positive multiples of 256).
// Returns 0, -1 for bad arguments, -2 if the launch failed.
extern "C" int ceiling_probe_store(int pattern, int32_t *C, int M, int N, hipStream_t stream)
{
    if (C == nullptr || M <= 0 || N <= 0 || M % 256 || N % 256 || pattern < 0 || pattern > 2 ||
        (int64_t)M * N > (int64_t(1) << 31))
        return -1;
    const void *fn = pattern == 0 ? (const void *)store_pattern<0>
                     : pattern == 1 ? (const void *)store_pattern<1>
                                    : (const void *)store_pattern<2>;
    const int lds = pattern == 2 ? 128 * (1024 + 16) : 0;
    if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return -2;
    int n = N;
    void *args[] = {&C, &n};
    if (hipLaunchKernel(fn, dim3((unsigned)((M / 256) * (N / 256))), dim3(512), args, lds, stream) != hipSuccess)
        return -2;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Work of one launch: operations (kinds 0-2, 4) or LDS bytes read (kind 3).
extern "C" double ceiling_probe_work(int kind, int blocks, int iters)
{
    const double per_block_iter =
        kind == 0 || kind == 2 ? 4.0 * kChains * 2 * 32 * 32 * 64      // 4 waves
        : kind == 1            ? 4.0 * kChains * 2 * 32 * 32 * 32
        : kind == 3            ? 8.0 * kFrags * kFrag                   // 8 waves
        : kind == 4            ? 8.0 * 8 * 2 * 32 * 32 * 64
                               : 0.0;
    return per_block_iter * blocks * iters;
}

// Floats of `out` one launch writes (one per thread).
extern "C" int64_t ceiling_probe_out_floats(int kind, int blocks)
{
    return (int64_t)blocks * threads_of(kind);
}

// Launch probe `kind` with `blocks` workgroups of `iters` iterations on
// `stream`; `out` is device memory of ceiling_probe_out_floats(kind, blocks)
// floats (`out_floats` says how many the caller has).  Returns 0, -1 for
// bad arguments, or -2 if the launch failed.
// `clocks`: NULL, or device memory of 2 * blocks int64 for each workgroup's
// shader-clock and constant-rate ticks over its loop.
extern "C" int ceiling_probe_run(int kind, int blocks, int iters, float *out, int64_t out_floats,
                                int64_t *clocks, hipStream_t stream)
{
    if (kind < 0 || kind > 4 || blocks < 1 || iters < 1 || out == nullptr ||
        out_floats < ceiling_probe_out_floats(kind, blocks))
        return -1;
    const void *fn = kind == 0   ? (const void *)mfma_loop<0>
                     : kind == 1 ? (const void *)mfma_loop<1>
                     : kind == 2 ? (const void *)mfma_loop<2>
                     : kind == 3 ? (const void *)lds_loop
                                 : (const void *)lds_mfma_loop;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsRequest) != hipSuccess)
        return -2;
    void *args[] = {&out, &iters, &clocks};
    if (hipLaunchKernel(fn, dim3((unsigned)blocks), dim3((unsigned)threads_of(kind)), args, kLdsRequest,
                        stream) != hipSuccess)
        return -2;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// The device's maximum shader clock, in kHz.
extern "C" int ceiling_probe_max_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
        return -1;
    return khz;
}

// Rate of the constant-rate counter read by the probes, in kHz.
extern "C" int ceiling_probe_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return -1;
    return khz;
}

// One configuration of the streaming-read family over `bytes` (a multiple of
// 1024, below 4 GiB, 16-byte aligned) at `buf`:
//   mode 0  buffer loads: `blocks` x `threads` threads, `inflight` in {1, 2,
//           4, 8} loads per thread, `policy` in {0, 1 (sc0), 2 (nt), 16 (sc1),
//           18 (sc1 nt)};
//   mode 1  direct-to-LDS: `blocks` x `threads` threads, `inflight` in {2, 4,
//           8, 16} 1 KB pieces per wave, `policy` 0 or 2 (nt); each workgroup
//           holds threads / 64 * inflight KB of LDS (at most 160 KB);
//   mode 2  direct-to-LDS in 64 KB strips (the narrow-M GEMM's pattern):
//           1024 threads, `inflight` 0 (one strip per workgroup, barrier per
//           strip), 4 or 8 pieces per wave, `policy` 2 (nt); `bytes` a
//           multiple of 64 KB.
// `out` holds at least blocks * threads ints.  Returns 0, -1 for arguments
// outside these sets, -2 if the launch failed.
extern "C" int ceiling_probe_stream_sweep(const void *buf, int64_t bytes, int mode, int blocks,
                                          int threads, int inflight, int policy, int32_t *out,
                                          int64_t out_ints, hipStream_t stream)
{
    if (buf == nullptr || out == nullptr || bytes <= 0 || (bytes & 1023) || bytes >= (int64_t(1) << 32) ||
        (reinterpret_cast<uintptr_t>(buf) & 15u) || blocks < 1 || threads < 64 || threads > 1024 ||
        (threads & 63) || out_ints < (int64_t)blocks * threads)
        return -1;
    const i32x4 rsrc = {(int32_t)(uint32_t)reinterpret_cast<uintptr_t>(buf),
                        (int32_t)((reinterpret_cast<uintptr_t>(buf) >> 32) & 0xFFFFu), (int32_t)bytes,
                        0x00020000};
    const void *fn = nullptr;
    int lds = 0;
    int64_t n = 0;
    if (mode == 0) {
        n = bytes / 16;
#define LPG_BUF(F, P) (inflight == F && policy == P) ? (const void *)stream_buf<F, P>
        fn = LPG_BUF(1, 0) : LPG_BUF(2, 0) : LPG_BUF(4, 0) : LPG_BUF(8, 0)
           : LPG_BUF(1, 1) : LPG_BUF(2, 1) : LPG_BUF(4, 1) : LPG_BUF(8, 1)
           : LPG_BUF(1, 2) : LPG_BUF(2, 2) : LPG_BUF(4, 2) : LPG_BUF(8, 2)
           : LPG_BUF(1, 16) : LPG_BUF(2, 16) : LPG_BUF(4, 16) : LPG_BUF(8, 16)
           : LPG_BUF(1, 18) : LPG_BUF(2, 18) : LPG_BUF(4, 18) : LPG_BUF(8, 18) : nullptr;
#undef LPG_BUF
    } else if (mode == 1) {
        n = bytes / 1024;
        lds = threads / 64 * inflight * 1024;
        if (lds > 160 * 1024) return -1;
#define LPG_DMA(F, P) (inflight == F && policy == (P ? 2 : 0)) ? (const void *)stream_dma<F, P>
        fn = LPG_DMA(2, false) : LPG_DMA(4, false) : LPG_DMA(8, false) : LPG_DMA(16, false)
           : LPG_DMA(2, true) : LPG_DMA(4, true) : LPG_DMA(8, true) : LPG_DMA(16, true) : nullptr;
#undef LPG_DMA
    } else if (mode == 2) {
        if (threads != 1024 || policy != 2 || (bytes & 65535)) return -1;
        n = bytes / 65536;
        lds = 16 * (inflight == 0 ? 4 : inflight) * 1024;
        fn = inflight == 0 ? (const void *)stream_strips<0>
           : inflight == 4 ? (const void *)stream_strips<4>
           : inflight == 8 ? (const void *)stream_strips<8> : nullptr;
    }
    if (fn == nullptr) return -1;
    if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return -2;
    i32x4 r = rsrc;
    int nbytes = (int)(uint32_t)bytes;
    void *args_buf[] = {const_cast<void **>(&buf), &nbytes, &n, &out};
    void *args_dma[] = {&r, &n, &out};
    void **args = mode == 0 ? args_buf : args_dma;
    if (hipLaunchKernel(fn, dim3((unsigned)blocks), dim3((unsigned)threads), args, lds, stream) != hipSuccess)
        return -2;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
