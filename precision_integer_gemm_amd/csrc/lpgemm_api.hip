// lpgemm_api.hip -- the C-ABI of the low-precision integer GEMM library:
// argument checks, kernel selection and launches (declarations and the full
// contract are in include/lpgemm.h).
#include "lpgemm.h"

#include <atomic>
#include <mutex>

#include "gemm_general.hpp"
#include "gemm_skinny.hpp"
#include "gemm_tiled.hpp"

using namespace lpgemm;

namespace {

std::atomic<int> g_override{LPGEMM_KERNEL_AUTO};

constexpr int kDefaultCUs = 256;  // MI355X
constexpr int kMaxDevices = 64;

// Compute units of the current device, queried once per device.
int device_cu_count()
{
    static std::once_flag once[kMaxDevices];
    static int cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    std::call_once(once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = kDefaultCUs;
        cus[dev] = n;
    });
    return cus[dev];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- kernel configurations -------------------------------------------------
// Tiled: 4 waves in 2 x 2, each wave 64 x 64 (2 x 2 blocks of 32 x 32), BK = 128.
template <int VAR>
using Tiled = TiledCfg<VAR, 2, 2, 2, 2, 128>;
#define TILED_KERNEL(VAR) gemm_tiled_kernel<VAR, 2, 2, 2, 2, 128>

// Skinny: strips of 32 rows of B, K split over 8 waves.
constexpr int kSkinnyFN = 2;
constexpr int kSkinnyKW = 8;
constexpr int kSkinnyMaxM = 16;

struct Plan {
    lpgemm_kernel kernel = LPGEMM_KERNEL_AUTO;
    int tile_m = 0, tile_n = 0, k_split = 1, threads = 0;
    int64_t workgroups = 0;
    int k_per_wave = 0;
    int tiles_n = 0;
};

lpgemm_status check_args(const void *A, const void *B, const void *C, int64_t M, int64_t N,
                         int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || (K & 1)) return LPGEMM_ERR_INVALID_ARG;
    if (K > LPGEMM_MAX_K) return LPGEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return LPGEMM_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return LPGEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
    return LPGEMM_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

lpgemm_status make_plan(lpgemm_variant variant, const void *A, const void *B, const void *C,
                        int64_t M, int64_t N, int64_t K, int cu_count, lpgemm_kernel forced,
                        Plan *plan)
{
    (void)cu_count;
    const bool fast_ok = (K % 32 == 0) && aligned16(A) && aligned16(B) && aligned16(C);
    const bool skinny_ok = fast_ok && variant == LPGEMM_VARIANT_W4A8 && M <= kSkinnyMaxM;

    lpgemm_kernel k = forced;
    if (k == LPGEMM_KERNEL_AUTO) {
        if (!fast_ok)
            k = LPGEMM_KERNEL_GENERAL;
        else if (skinny_ok)
            k = LPGEMM_KERNEL_SKINNY;
        else
            k = LPGEMM_KERNEL_TILED;
    }
    if ((k == LPGEMM_KERNEL_TILED && !fast_ok) || (k == LPGEMM_KERNEL_SKINNY && !skinny_ok))
        return LPGEMM_ERR_UNSUPPORTED;

    Plan p;
    p.kernel = k;
    switch (k) {
    case LPGEMM_KERNEL_GENERAL:
        p.tile_m = 16;
        p.tile_n = 16;
        p.threads = 256;
        p.workgroups = ceil_div(M, 16) * ceil_div(N, 16);
        if (ceil_div(M, 16) > 65535 || ceil_div(N, 16) > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        break;
    case LPGEMM_KERNEL_TILED: {
        const int bm = (variant == LPGEMM_VARIANT_I4I4) ? Tiled<I4I4>::BM : Tiled<W4A8>::BM;
        const int bn = (variant == LPGEMM_VARIANT_I4I4) ? Tiled<I4I4>::BN : Tiled<W4A8>::BN;
        p.tile_m = bm;
        p.tile_n = bn;
        p.threads = Tiled<I4I4>::kThreads;
        p.tiles_n = (int)ceil_div(N, bn);
        p.workgroups = ceil_div(M, bm) * p.tiles_n;
        if (p.workgroups > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        break;
    }
    case LPGEMM_KERNEL_SKINNY: {
        p.tile_m = kSkinnyMaxM;
        p.tile_n = kSkinnyFN * 16;
        p.k_split = kSkinnyKW;
        p.threads = 64 * kSkinnyKW;
        p.k_per_wave = (int)(ceil_div(ceil_div(K, kSkinnyKW), 128) * 128);
        p.workgroups = ceil_div(N, p.tile_n);
        break;
    }
    default:
        return LPGEMM_ERR_INVALID_ARG;
    }
    *plan = p;
    return LPGEMM_OK;
}

lpgemm_status launched()
{
    return hipGetLastError() == hipSuccess ? LPGEMM_OK : LPGEMM_ERR_HIP;
}

lpgemm_status run_gemm(lpgemm_variant variant, const void *A, const void *B, int32_t *C,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    lpgemm_status st = check_args(A, B, C, M, N, K);
    if (st != LPGEMM_OK || M == 0 || N == 0) return st;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (K == 0) {
        const int64_t count = M * N;
        const int blocks = (int)std::min<int64_t>(ceil_div(count, 256), 65536);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, C, count);
        return launched();
    }
    Plan p;
    st = make_plan(variant, A, B, C, M, N, K, device_cu_count(),
                   (lpgemm_kernel)g_override.load(std::memory_order_relaxed), &p);
    if (st != LPGEMM_OK) return st;

    const uint8_t *a = static_cast<const uint8_t *>(A);
    const uint8_t *b = static_cast<const uint8_t *>(B);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (p.kernel) {
    case LPGEMM_KERNEL_GENERAL: {
        const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16));
        if (variant == LPGEMM_VARIANT_I4I4)
            hipLaunchKernelGGL(gemm_general_kernel<I4I4>, grid, dim3(256), 0, stream, a, b, C, M, N, K);
        else
            hipLaunchKernelGGL(gemm_general_kernel<W4A8>, grid, dim3(256), 0, stream, a, b, C, M, N, K);
        break;
    }
    case LPGEMM_KERNEL_TILED:
        if (variant == LPGEMM_VARIANT_I4I4)
            hipLaunchKernelGGL(TILED_KERNEL(I4I4), dim3((unsigned)p.workgroups),
                               dim3(Tiled<I4I4>::kThreads), Tiled<I4I4>::LDS_BYTES, stream, a, b, C,
                               m, n, k, p.tiles_n);
        else
            hipLaunchKernelGGL(TILED_KERNEL(W4A8), dim3((unsigned)p.workgroups),
                               dim3(Tiled<W4A8>::kThreads), Tiled<W4A8>::LDS_BYTES, stream, a, b, C,
                               m, n, k, p.tiles_n);
        break;
    case LPGEMM_KERNEL_SKINNY:
        hipLaunchKernelGGL((gemm_w4a8_skinny_kernel<kSkinnyFN, kSkinnyKW>),
                           dim3((unsigned)p.workgroups), dim3(p.threads), 0, stream,
                           static_cast<const int8_t *>(A), b, C, m, n, k, p.k_per_wave);
        break;
    default:
        return LPGEMM_ERR_INVALID_ARG;
    }
    return launched();
}

lpgemm_status run_elementwise(bool pack, const void *src, void *dst, int64_t rows, int64_t K,
                              hipStream_t stream)
{
    if (rows < 0 || K < 0 || (K & 1)) return LPGEMM_ERR_INVALID_ARG;
    const int64_t bytes = rows * (K / 2);
    if (bytes == 0) return LPGEMM_OK;
    if (src == nullptr || dst == nullptr) return LPGEMM_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const int blocks = (int)std::min<int64_t>(ceil_div(bytes, 256), 65536);
    if (pack)
        hipLaunchKernelGGL(pack_int4_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const int8_t *>(src), static_cast<uint8_t *>(dst), bytes);
    else
        hipLaunchKernelGGL(unpack_int4_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint8_t *>(src), static_cast<int8_t *>(dst), bytes);
    return launched();
}

}  // namespace

extern "C" {

lpgemm_status lpgemm_int4_int4(const void *A_packed, const void *B_packed, int32_t *C, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream)
{
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, M, N, K, stream);
}

lpgemm_status lpgemm_w4a8(const int8_t *A, const uint8_t *B_packed, int32_t *C, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    return run_gemm(LPGEMM_VARIANT_W4A8, A, B_packed, C, M, N, K, stream);
}

lpgemm_status lpgemm_pack_int4(const int8_t *logical, uint8_t *packed, int64_t rows, int64_t K,
                               hipStream_t stream)
{
    return run_elementwise(true, logical, packed, rows, K, stream);
}

lpgemm_status lpgemm_unpack_int4(const uint8_t *packed, int8_t *logical, int64_t rows, int64_t K,
                                 hipStream_t stream)
{
    return run_elementwise(false, packed, logical, rows, K, stream);
}

const char *lpgemm_status_string(lpgemm_status status)
{
    switch (status) {
    case LPGEMM_OK: return "ok";
    case LPGEMM_ERR_INVALID_ARG: return "invalid argument";
    case LPGEMM_ERR_UNSUPPORTED: return "unsupported";
    case LPGEMM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

lpgemm_status lpgemm_plan(lpgemm_variant variant, const void *A, const void *B, const void *C,
                          int64_t M, int64_t N, int64_t K, int32_t cu_count,
                          lpgemm_plan_info *info)
{
    if (info == nullptr || (variant != LPGEMM_VARIANT_I4I4 && variant != LPGEMM_VARIANT_W4A8))
        return LPGEMM_ERR_INVALID_ARG;
    lpgemm_status st = check_args(A, B, C, M, N, K);
    if (st != LPGEMM_OK) return st;
    *info = lpgemm_plan_info{};
    if (M == 0 || N == 0 || K == 0) return LPGEMM_OK;  // nothing, or a zero fill
    Plan p;
    st = make_plan(variant, A, B, C, M, N, K, cu_count > 0 ? cu_count : kDefaultCUs,
                   (lpgemm_kernel)g_override.load(std::memory_order_relaxed), &p);
    if (st != LPGEMM_OK) return st;
    info->kernel = p.kernel;
    info->tile_m = p.tile_m;
    info->tile_n = p.tile_n;
    info->k_split = p.k_split;
    info->workgroups = p.workgroups;
    info->threads = p.threads;
    return LPGEMM_OK;
}

lpgemm_status lpgemm_set_kernel_override(lpgemm_kernel kernel)
{
    if (kernel < LPGEMM_KERNEL_AUTO || kernel > LPGEMM_KERNEL_SKINNY) return LPGEMM_ERR_INVALID_ARG;
    g_override.store(kernel, std::memory_order_relaxed);
    return LPGEMM_OK;
}

}  // extern "C"
