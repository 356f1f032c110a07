// Drives the host-side paths of the library -- argument checks, planning,
// workspace sizing, the scratch-limit check -- over a wide grid of shapes and
// arguments, for a host-only build with AddressSanitizer and
// UndefinedBehaviorSanitizer (signed overflow in the size arithmetic, for
// instance, aborts the run).  No call here reaches a kernel launch: every
// shape is planned, and the entry points are called only with arguments they
// reject before any HIP call.  Exit status 0 when all checks pass.
#include <cstdint>
#include <cstdio>

#include "lpgemm.h"

static int failures = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main()
{
    const int64_t sizes[] = {0, 1, 2, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000,
                             1024, 3000, 4096, 5120, 8192, 16384, 28672, 65536, 1 << 20,
                             (int64_t)INT32_MAX, (int64_t)INT32_MAX + 1, INT64_MAX / 4};
    const int64_t ks[] = {-2, 0, 2, 30, 32, 34, 64, 96, 1024, 2048, 3072, 4096, 6144, 8192, 8224,
                          12288, 28672, 65536, 131040, 131070, 131072, 1 << 30};
    const int cus[] = {0, 1, 8, 80, 256, 304, 1024};
    const lpgemm_kernel kernels[] = {LPGEMM_KERNEL_AUTO, LPGEMM_KERNEL_GENERAL, LPGEMM_KERNEL_TILED,
                                     LPGEMM_KERNEL_SKINNY, LPGEMM_KERNEL_TILED_128,
                                     LPGEMM_KERNEL_TILED_256, LPGEMM_KERNEL_TILED_64,
                                     LPGEMM_KERNEL_FP6};
    const void *P = reinterpret_cast<const void *>(uintptr_t{4096});
    const void *U = reinterpret_cast<const void *>(uintptr_t{4097});
    const size_t wss[] = {0, 1000, size_t(1) << 26, SIZE_MAX};
    long planned = 0;
    for (lpgemm_kernel kern : kernels) {
        CHECK(lpgemm_set_kernel_override(kern) == LPGEMM_OK);
        for (int v = 0; v < 2; ++v)
            for (int64_t M : sizes)
                for (int64_t N : sizes)
                    for (int64_t K : ks)
                        for (int cu : cus)
                            for (size_t ws : wss) {
                                if ((cu != 256 && cu != 0) && ws != SIZE_MAX) continue;
                                lpgemm_plan_info info{};
                                const lpgemm_status st = lpgemm_plan((lpgemm_variant)v, P, (M & 1) ? U : P, P,
                                                                     M, N, K, ws, cu, &info);
                                CHECK(st == LPGEMM_OK || st == LPGEMM_ERR_INVALID_ARG ||
                                      st == LPGEMM_ERR_UNSUPPORTED);
                                if (st == LPGEMM_OK && M > 0 && N > 0 && K > 0) {
                                    CHECK(info.workgroups >= 1 && info.threads >= 64);
                                    CHECK(info.k_chunks >= 1);
                                    CHECK((uint64_t)info.workspace_bytes <= ws);
                                }
                                ++planned;
                            }
    }
    CHECK(lpgemm_set_kernel_override(LPGEMM_KERNEL_AUTO) == LPGEMM_OK);
    CHECK(lpgemm_set_kernel_override((lpgemm_kernel)99) == LPGEMM_ERR_INVALID_ARG);
    // workspace sizes
    for (int v = 0; v < 2; ++v)
        for (int scaled = 0; scaled < 2; ++scaled)
            for (int64_t M : sizes)
                for (int64_t N : sizes)
                    for (int64_t K : ks) {
                        size_t b = 7;
                        const lpgemm_status st = lpgemm_workspace_size((lpgemm_variant)v, scaled, M, N, K, 0, &b);
                        CHECK(st == LPGEMM_OK || st == LPGEMM_ERR_INVALID_ARG || st == LPGEMM_ERR_UNSUPPORTED);
                        if (st == LPGEMM_OK && (M == 0 || N == 0 || K == 0)) CHECK(b == 0);
                    }
    size_t b = 0;
    CHECK(lpgemm_workspace_size((lpgemm_variant)2, 0, 4, 4, 32, 0, &b) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_workspace_size(LPGEMM_VARIANT_I4I4, 0, 4, 4, 32, 0, nullptr) == LPGEMM_ERR_INVALID_ARG);
    // entry points: arguments rejected before any HIP call
    int32_t *C = (int32_t *)P;
    void *W = const_cast<void *>(P);
    for (int64_t K : {-2L, 33L, 131072L}) {
        CHECK(lpgemm_int4_int4(P, P, C, 4, 4, K, nullptr) != LPGEMM_OK);
        CHECK(lpgemm_w4a8((const int8_t *)P, (const uint8_t *)P, C, 4, 4, K, nullptr) != LPGEMM_OK);
        CHECK(lpgemm_int4_int4_ws(P, P, C, 4, 4, K, W, 4096, nullptr) != LPGEMM_OK);
        CHECK(lpgemm_w4a8_ws((const int8_t *)P, (const uint8_t *)P, C, 4, 4, K, W, 4096, nullptr) != LPGEMM_OK);
        CHECK(lpgemm_int4_int4_noalloc(P, P, C, 4, 4, K, nullptr) != LPGEMM_OK);
        CHECK(lpgemm_fp8_e4m3((const uint8_t *)P, (const uint8_t *)P, C, LPGEMM_OUT_F32, 4, 4, K < 0 ? K : 131071,
                              nullptr) != LPGEMM_OK);
        CHECK(lpgemm_fp8_e5m2((const uint8_t *)P, (const uint8_t *)P, C, LPGEMM_OUT_F32, 4, 4, K < 0 ? K : 131071,
                              nullptr) != LPGEMM_OK);
    }
    CHECK(lpgemm_int4_int4(P, P, nullptr, 4, 4, 32, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_ws(P, P, C, 4, 4, 32, nullptr, 64, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_ws(P, P, C, 4, 4, 32, (char *)W + 8, 64, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_scaled(P, P, nullptr, (const float *)P, W, LPGEMM_OUT_BF16, 4, 4, 32, nullptr) ==
          LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_w4a8_scaled((const int8_t *)P, (const uint8_t *)P, (const float *)P, (const float *)P, W,
                             (lpgemm_out_dtype)9, 4, 4, 32, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_scaled_ws(P, P, (const float *)P, (const float *)P, W, LPGEMM_OUT_FP8_E4M3, 4, 4,
                                     32, nullptr, 0, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_fp8_e5m2((const uint8_t *)P, (const uint8_t *)P, C, LPGEMM_OUT_FP8_E4M3, 4, 4, 16, nullptr) ==
          LPGEMM_ERR_INVALID_ARG);
    // block-scaled products: every argument error before any HIP call
    const float *F = (const float *)P;
    for (int64_t g : {0L, 16L, 48L, 100L, (int64_t)1 << 31})
        CHECK(lpgemm_int4_int4_blockscaled(P, P, F, F, g, W, LPGEMM_OUT_F32, 4, 4, 64, nullptr) ==
              LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_w4a8_blockscaled((const int8_t *)P, (const uint8_t *)P, F, F, 32, W, LPGEMM_OUT_FP8_E4M3, 4, 4,
                                  64, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_w4a8_blockscaled((const int8_t *)P, (const uint8_t *)P, F, F, 32, W, LPGEMM_OUT_F32, 4, 4, 63,
                                  nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_blockscaled(P, P, nullptr, F, 32, W, LPGEMM_OUT_BF16, 4, 4, 64, nullptr) ==
          LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_blockscaled(P, P, F, (const float *)((const char *)P + 2), 32, W, LPGEMM_OUT_BF16, 4, 4,
                                       64, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_blockscaled(P, P, F, F, 32, (char *)W + 1, LPGEMM_OUT_F16, 4, 4, 64, nullptr) ==
          LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_int4_int4_blockscaled(P, P, F, F, 32, W, LPGEMM_OUT_F32, 4, 4, 131072, nullptr) ==
          LPGEMM_ERR_UNSUPPORTED);
    CHECK(lpgemm_int4_int4_blockscaled(P, P, F, F, 32, W, LPGEMM_OUT_F32, 0, 4, 64, nullptr) == LPGEMM_OK);
    CHECK(lpgemm_fp8_e4m3((const uint8_t *)P, (const uint8_t *)P, C, LPGEMM_OUT_FP8_E5M2, 4, 4, 16, nullptr) ==
          LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_pack_int4((const int8_t *)P, (uint8_t *)W, 3, 5, nullptr) == LPGEMM_ERR_INVALID_ARG);
    CHECK(lpgemm_unpack_int4((const uint8_t *)P, (int8_t *)W, INT64_MAX, 4, nullptr) == LPGEMM_ERR_UNSUPPORTED);
    // the scratch limit of the allocation-free entry point, before any launch
    CHECK(lpgemm_int4_int4_noalloc(P, P, C, 16384, 16384, 8192, nullptr) == LPGEMM_ERR_SCRATCH_LIMIT);
    // empty products are no-ops
    CHECK(lpgemm_int4_int4(nullptr, nullptr, nullptr, 0, 4, 32, nullptr) == LPGEMM_OK);
    CHECK(lpgemm_int4_int4_noalloc(nullptr, nullptr, nullptr, 4, 0, 32, nullptr) == LPGEMM_OK);
    for (int s = -1; s < 6; ++s) CHECK(lpgemm_status_string((lpgemm_status)s) != nullptr);
    if (failures)
        std::fprintf(stderr, "%d checks failed\n", failures);
    else
        std::printf("host-path sanitizer run: %ld plans, all checks passed\n", planned);
    return failures ? 1 : 0;
}
