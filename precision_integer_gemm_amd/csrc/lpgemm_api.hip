// lpgemm_api.hip -- the C-ABI of the low-precision integer GEMM library:
// argument checks, kernel selection and launches (declarations and the full
// contract are in include/lpgemm.h).
#include "lpgemm.h"

#include <cmath>
#include <mutex>

#include "gemm_general.hpp"
#include "gemm_skinny.hpp"
#include "gemm_pipelined.hpp"
#include "gemm_fp6.hpp"

using namespace lpgemm;

namespace {

// Kernel forced by lpgemm_set_kernel_override for calls made on this thread.
thread_local int t_override = LPGEMM_KERNEL_AUTO;

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
// Tiled kernels (gemm_pipelined.hpp), chosen by measurement on MI355X:
//   large: 256 x 256 tiles, 8 waves (2 x 4), each wave 128 (m) x 64 (n);
//          int4 x int4 stages 256 logical k per LDS slot (2 slots, 128 KB),
//          W4A8 128 k per slot (2 slots, 96 KB: a third slot measured
//          1-4% slower).
//   tiny:  64 x 64 tiles, 4 waves, when even 128 x 128 tiles would leave
//          more than half of the compute units idle (1024^3: 64 -> 256 tiles).
//   small: 128 x 128 tiles, 4 waves, for shapes with too few large tiles to
//          fill the GPU.
template <int VAR, int FM, int FN, int WM, int WN, int BK, int ST>
struct TiledKernel {
    using Cfg = PipeCfg<VAR, FM, FN, WM, WN, BK, ST>;
    template <int OUT, bool SPLIT = false>
    static void *fn() { return reinterpret_cast<void *>(&gemm_pipelined_kernel<VAR, FM, FN, WM, WN, BK, ST, OUT, SPLIT>); }
};
using I4Large = TiledKernel<I4I4, 4, 2, 2, 4, 256, 2>;
using W8Large = TiledKernel<W4A8, 4, 2, 2, 4, 128, 2>;
using I4Small = TiledKernel<I4I4, 2, 2, 2, 2, 128, 3>;
using W8Small = TiledKernel<W4A8, 2, 2, 2, 2, 128, 3>;
using I4Tiny = TiledKernel<I4I4, 1, 1, 2, 2, 256, 2>;
using W8Tiny = TiledKernel<W4A8, 1, 1, 2, 2, 256, 2>;
// fp8 (FP8: e4m3, BF8: e5m2): one byte per element on both operands, the
// W4A8 kernel's A side for both; 128 k per LDS stage.
template <int VAR> using F8Large = TiledKernel<VAR, 4, 2, 2, 4, 128, 2>;
template <int VAR> using F8Small = TiledKernel<VAR, 2, 2, 2, 2, 128, 3>;
template <int VAR> using F8Tiny = TiledKernel<VAR, 1, 1, 2, 2, 128, 2>;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs

// FP6 path (gemm_fp6.hpp): 256 x 256 tiles, 8 waves of 128 (m) x 64 (n), three
// LDS stages of 128 k (144 KB), after one launch that re-encodes both
// operands.  Chosen automatically for int4 x int4 where the re-encoding pays
// for itself, measured against the int8 tiled kernel (interleaved, outputs
// identical): with the 256-tiles covering three quarters of the compute units
// and K >= 3072 (3000 x 5120 x 6144, 240 tiles: 89.0 -> 78.0 us; 4096^3 64.9
// -> 60.5; 4096 x 3584 x 4096 +9%; 2560 x 5120 x 8192 +17%), or two tiles
// per compute unit and K >= 2048 (8192^2 x 2048 +20%, 8192^3 472 -> 371 us);
// not below (4096^2 x 2048 even; 3072^2 x 4096, 144 tiles, +2.5%;
// 2048 x 4096 x 4096, 128 tiles, -14%; 2048^2 x 8192 -38%).
constexpr int kFp6FM = 4, kFp6FN = 2, kFp6WM = 2, kFp6WN = 4, kFp6KS = 2, kFp6Stages = 3;
using Fp6Tile = Fp6Cfg<kFp6FM, kFp6FN, kFp6WM, kFp6WN, kFp6KS, kFp6Stages>;
constexpr int64_t kFp6MinK = 2048, kFp6OneTileK = 3072;

// Up to this many rows of A the product is bound by reading B once: no
// 256-tiles and no FP6 re-encoding (which alone moves 2.5x B's bytes).  With
// 64 x 65536 x 8192 int4 operands the FP6 path took 263 us against 80 us on
// 64- or 128-tiles; with W4A8 64 x 65536 x 4096, 256-tiles 58 us against 48.
constexpr int64_t kSmallM = 128;
// Split 64-tile (and very few 128-tile) calls: K of at least kTiledSplitK,
// ranges of at least kTiledMinRange.
constexpr int64_t kTiledMinRange = 1024, kTiledSplitK = 12288;

bool fp6_pays(int64_t K, int64_t tiles256, int cu_count)
{
    return (K >= kFp6MinK && tiles256 >= 2 * (int64_t)cu_count) ||
           (K >= kFp6OneTileK && 4 * tiles256 >= 3 * (int64_t)cu_count);
}

// Skinny (both formats, M <= 16): 16 waves split K (up to 4 steps of 128 k
// each, A held in registers);
// one workgroup per compute unit walks strips of 16 rows of B, staged in LDS.
// (16 waves contract a strip faster than 8 with twice the steps each.)  Longer
// K (int32 output) is cut into equal ranges of at most kSkinnyMaxK, a multiple
// of 256, each taken by its own group of workgroups and added into C.
// Up to kSkinnyMaxM rows run as row groups of 16 (each group's workgroups
// stream every strip; the other groups' reads hit L2 / MALL).  The automatic
// choice takes the kernel up to kSkinnyAutoM rows, and up to kSkinnyMaxM rows
// when K needs several K ranges or 64-tiles would not fill the compute units
// (measured: 32 x 8192 x 28672 107 -> 53 us, 32 x 4096 x 4096 20 -> 15 us; at
// 48-64 x 28672 x 8192 the row groups lose to 64-tiles, 52-60 against 41-47 us).
constexpr int kSkinnyKW = 16;
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnyAutoM = 16;
constexpr int kSkinnyMaxK = kSkinnyKW * 4 * 128;

struct Plan {
    lpgemm_kernel kernel = LPGEMM_KERNEL_AUTO;
    int tile_m = 0, tile_n = 0, k_split = 1, threads = 0;
    int64_t workgroups = 0;
    int k_steps = 0;
    int k_chunks = 1, kc = 0;  // K ranges, and their length
    bool k_seq = false;        // skinny: each workgroup takes every range of its strips
    int tiles_m = 0, tiles_n = 0;
    int tile = 0;  // tiled kernels: 256, 128 or 64 (square tiles)
    int64_t ws_bytes = 0;  // workspace the launch uses (FP6 copies or K-range slices)
};

constexpr uint64_t kWsAlign = 256;  // workspace base alignment, and of the B copy inside it
uint64_t align_ws(uint64_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace of the FP6 path: A's FP6 copy (padded to kWsAlign), then B's.
int64_t fp6_workspace(int64_t M, int64_t N, int64_t K)
{
    return (int64_t)align_ws((uint64_t)fp6_bytes(M, K)) + fp6_bytes(N, K);
}

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

// Narrow-M workgroups per row group (of `sets` sets sharing the compute
// units); with several row groups a multiple of 8, which keeps the sets that
// read one strip on one XCD.
int64_t skinny_per_set(int64_t M, int64_t N, int64_t sets, int cu_count)
{
    int64_t per_set = std::min<int64_t>(ceil_div(N, 16),
                                        std::max<int64_t>(1, std::min(cu_count, 256) / sets));
    if (ceil_div(M, 16) > 1 && per_set >= 8) per_set -= per_set % 8;
    return per_set;
}

// K ranges taken range by range inside each workgroup (no zero fill, no
// atomics: the path of the scaled formats with long K) when every workgroup of
// a row group gets at most kSkinnyKW strips and the strips keep at least half
// of the compute units busy.
bool skinny_seq_fits(int64_t M, int64_t N, int cu_count)
{
    const int64_t strips = ceil_div(N, 16);
    const int64_t per = skinny_per_set(M, N, ceil_div(M, 16), cu_count);
    return ceil_div(strips, per) <= kSkinnyKW && strips * 2 >= std::min(cu_count, 256);
}

// int_out: the result is the int32 C (split K is available), not a scaled one.
// ws_bytes: the workspace the caller provides; paths that need more are not
// taken (a forced FP6 kernel is then unsupported), and K ranges are limited to
// the slices that fit.
lpgemm_status make_plan(lpgemm_variant variant, const void *A, const void *B, const void *C,
                        int64_t M, int64_t N, int64_t K, int cu_count, lpgemm_kernel forced,
                        bool int_out, uint64_t ws_bytes, Plan *plan)
{
    const bool fast_ok = (K % 32 == 0) && aligned16(A) && aligned16(B) && aligned16(C);
    const bool skinny_ok = fast_ok && M <= kSkinnyMaxM &&
                           (K <= kSkinnyMaxK || int_out || skinny_seq_fits(M, N, cu_count)) &&
                           N * (K / 2) < INT32_MAX;

    const bool fp6_ok = fast_ok && variant == LPGEMM_VARIANT_I4I4;
    const bool fp6_ws = (uint64_t)fp6_workspace(M, N, K) <= ws_bytes;
    const int64_t large_tiles = ceil_div(M, 256) * ceil_div(N, 256);

    lpgemm_kernel k = forced;
    if (k == LPGEMM_KERNEL_AUTO) {
        if (!fast_ok)
            k = LPGEMM_KERNEL_GENERAL;
        else if (skinny_ok && (M <= kSkinnyAutoM || K > kSkinnyMaxK ||
                               ceil_div(M, 64) * ceil_div(N, 64) < cu_count))
            k = LPGEMM_KERNEL_SKINNY;
        else if (fp6_ok && fp6_ws && M > kSmallM && fp6_pays(K, large_tiles, cu_count))
            k = LPGEMM_KERNEL_FP6;
        else
            k = LPGEMM_KERNEL_TILED;
    }
    const bool tiled = k == LPGEMM_KERNEL_TILED || k == LPGEMM_KERNEL_TILED_128 ||
                       k == LPGEMM_KERNEL_TILED_256 || k == LPGEMM_KERNEL_TILED_64;
    if ((tiled && !fast_ok) || (k == LPGEMM_KERNEL_SKINNY && !skinny_ok) ||
        (k == LPGEMM_KERNEL_FP6 && !(fp6_ok && fp6_ws)))
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
    case LPGEMM_KERNEL_TILED:
    case LPGEMM_KERNEL_TILED_128:
    case LPGEMM_KERNEL_TILED_256:
    case LPGEMM_KERNEL_TILED_64: {
        // Large tiles when they give at least 3/4 of a tile per compute unit;
        // else 128-tiles when they number at least the compute units; else
        // 64-tiles (two run on a compute unit at once, so they beat 128-tiles
        // that leave compute units idle: 256 x 8192 x 8192 19-24% faster).
        // Up to kSmallM rows (one row of 128-tiles, B read once) never
        // 256-tiles, mostly empty there; from 65 rows 64-tiles would read B
        // twice, so 128-tiles already when they cover half the compute units.
        const int64_t small_tiles = ceil_div(M, 128) * ceil_div(N, 128);
        if (k == LPGEMM_KERNEL_TILED) {
            if (M <= 64)
                p.tile = small_tiles >= (int64_t)cu_count ? 128 : 64;
            else if (M <= kSmallM)
                p.tile = small_tiles * 2 >= (int64_t)cu_count ? 128 : 64;
            else
                p.tile = large_tiles * 4 >= (int64_t)cu_count * 3 ? 256
                         : small_tiles >= (int64_t)cu_count       ? 128
                                                                  : 64;
        }
        else
            p.tile = k == LPGEMM_KERNEL_TILED_256 ? 256 : k == LPGEMM_KERNEL_TILED_128 ? 128 : 64;
        p.kernel = LPGEMM_KERNEL_TILED;
        p.tile_m = p.tile;
        p.tile_n = p.tile;
        p.threads = p.tile == 256 ? I4Large::Cfg::kThreads
                    : p.tile == 128 ? I4Small::Cfg::kThreads
                                    : I4Tiny::Cfg::kThreads;
        p.tiles_m = (int)ceil_div(M, p.tile_m);
        p.tiles_n = (int)ceil_div(N, p.tile_n);
        p.workgroups = (int64_t)p.tiles_m * p.tiles_n;
        if (p.workgroups > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        // Automatic 64-tiles too few for two per compute unit, with K of at
        // least kTiledSplitK (int32 result): S K ranges of at least
        // kTiledMinRange, each storing its partial tiles into its own M x N
        // int32 workspace slice, summed into C by a second kernel; at most two
        // workgroups per compute unit, S = 35 sqrt(K / (M N)) (the longest
        // range against the slices' 2 S M N words).  Measured on MI355X, one
        // range -> S ranges (W4A8): 128 x 8192 x 28672 113 -> 82 us (S = 2),
        // 96 x 4096 x 14336 48 -> 40 us, 128 x 2048 x 65536 164 -> 53 us,
        // 100 x 700 x 65536 163 -> 40 us, 200 x 100 x 131040 376 -> 53 us; at
        // K = 8192 (130 x 1000) the workspace and the second kernel cost more
        // (29 -> 38 us), hence the K bound.  Adding the ranges into C with
        // int32 atomics instead costs about 17 us per million adds.  Automatic
        // 128-tiles split only when fewer than two thirds of the compute units
        // have one: 128 x 16384 x 28672 (128 tiles) 158 -> 99 us W4A8, 118 ->
        // 92 us int4; 96 x 20000 x 16384 (157 tiles) 90 -> 76 us W4A8, even for
        // int4; from 224 tiles on the single range is faster (100 x 28672 x
        // 14336: 84 against 90 us).
        const bool split_tile = p.tile == 64 || (p.tile == 128 && 3 * p.workgroups < 2 * (int64_t)cu_count);
        if (k == LPGEMM_KERNEL_TILED && int_out && split_tile &&
            p.workgroups < 2 * (int64_t)cu_count && K >= kTiledSplitK) {
            const double mn = (double)M * (double)N;
            int64_t chunks = std::llround(35.0 * std::sqrt((double)K / mn));
            chunks = std::max<int64_t>(2, std::min<int64_t>(
                chunks, std::min<int64_t>(ceil_div(2 * (int64_t)cu_count, p.workgroups),
                                          K / kTiledMinRange)));
            // no more ranges than the workspace has slices for (none below two)
            const uint64_t slice = (uint64_t)M * (uint64_t)N * 4u;
            chunks = std::min<int64_t>(chunks, (int64_t)std::min<uint64_t>(ws_bytes / slice, 1u << 20));
            const int64_t kc = ceil_div(ceil_div(K, std::max<int64_t>(chunks, 1)), 256) * 256;
            chunks = ceil_div(K, kc);
            if (chunks >= 2) {
                p.k_chunks = (int)chunks;
                p.kc = (int)kc;
                p.workgroups *= chunks;
                p.ws_bytes = (int64_t)(chunks * slice);
            }
        }
        // Large tiles run one persistent workgroup per compute unit (their LDS
        // ring leaves room for one), each looping over tiles.
        if (p.tile == 256) p.workgroups = std::min<int64_t>(p.workgroups, cu_count);
        break;
    }
    case LPGEMM_KERNEL_FP6: {
        p.tile = 256;
        p.tile_m = Fp6Tile::BM;
        p.tile_n = Fp6Tile::BN;
        p.threads = Fp6Tile::kThreads;
        p.tiles_m = (int)ceil_div(M, Fp6Tile::BM);
        p.tiles_n = (int)ceil_div(N, Fp6Tile::BN);
        if ((int64_t)p.tiles_m * p.tiles_n > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        // the conversion grid: one workgroup per row block and kFp6ConvWaves k blocks
        if ((ceil_div(M, 32) + ceil_div(N, 32)) * ceil_div(ceil_div(K, 64), kFp6ConvWaves) > INT32_MAX)
            return LPGEMM_ERR_UNSUPPORTED;
        p.workgroups = std::min<int64_t>((int64_t)p.tiles_m * p.tiles_n, cu_count);
        p.ws_bytes = fp6_workspace(M, N, K);
        break;
    }
    case LPGEMM_KERNEL_SKINNY: {
        p.tile_m = 16;  // rows per group
        p.tile_n = 16;
        p.k_split = kSkinnyKW;
        p.threads = 64 * kSkinnyKW;
        int64_t chunks = ceil_div(K, kSkinnyMaxK);
        const int64_t kc = chunks > 1 ? ceil_div(ceil_div(K, chunks), 256) * 256 : K;
        chunks = ceil_div(K, kc);
        p.k_chunks = (int)chunks;
        p.kc = (int)kc;
        p.k_steps = (int)ceil_div(ceil_div(kc, kSkinnyKW), 128);  // 1..4
        while (p.k_steps & (p.k_steps - 1)) ++p.k_steps;           // 1, 2 or 4
        // sets of workgroups: row groups x K ranges, or row groups alone when
        // each workgroup takes every range of its strips
        const int64_t mgroups = ceil_div(M, 16);
        // (int32 results add their ranges into C: measured faster than taking
        // the ranges in turn, 38.1 against 42.3 us at 16 x 8192 x 28672)
        p.k_seq = chunks > 1 && !int_out && skinny_seq_fits(M, N, cu_count);
        const int64_t sets = p.k_seq ? mgroups : mgroups * chunks;
        p.workgroups = sets * skinny_per_set(M, N, sets, cu_count);
        break;
    }
    default:
        return LPGEMM_ERR_INVALID_ARG;
    }
    *plan = p;
    return LPGEMM_OK;
}

// Scratch of the allocation-free entry point (lpgemm_int4_int4_noalloc): a
// file-scope device array, one copy per device, held from the library's load
// on that device until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in): the device address
// comes from static_scratch().
static __device__ __align__(256) uint8_t scratch[LPGEMM_STATIC_SCRATCH_BYTES];

// This device's address of `scratch`, looked up once per device with that
// device current.
lpgemm_status static_scratch(void **ptr)
{
    static std::once_flag once[kMaxDevices];
    static void *addr[kMaxDevices];
    static hipError_t err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        void *p = nullptr;
        err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err[dev] == hipSuccess && p == nullptr) err[dev] = hipErrorInvalidSymbol;
        addr[dev] = p;
    });
    if (err[dev] != hipSuccess) return LPGEMM_ERR_HIP;
    *ptr = addr[dev];
    return LPGEMM_OK;
}

lpgemm_status launched()
{
    return hipGetLastError() == hipSuccess ? LPGEMM_OK : LPGEMM_ERR_HIP;
}

// Launch a tiled configuration; the first launch on each device raises the
// kernel's dynamic-LDS limit to the ring size (above the 64 KB default).
// SPLIT: the plan's K ranges, each storing its partial tiles into its own
// M x N int32 slice of the caller's workspace `ws`; a second kernel sums the
// slices into C.
template <class TK, int OUT, bool SPLIT = false>
lpgemm_status launch_tiled(const Plan &p, const uint8_t *a, const uint8_t *b, Epilogue epi, int m,
                           int n, int k, void *ws, hipStream_t stream)
{
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        attr_err[dev] = hipFuncSetAttribute(TK::template fn<OUT, SPLIT>(),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            TK::Cfg::LDS_BYTES);
    });
    if (attr_err[dev] != hipSuccess) return LPGEMM_ERR_HIP;
    int tiles_m = p.tiles_m, tiles_n = p.tiles_n, xcds = kXcds;
    int kc = SPLIT ? p.kc : k;
    Epilogue e_gemm = epi;
    const int64_t count = (int64_t)m * n;
    if (SPLIT) {  // one int32 M x N slice per K range
        if (ws == nullptr) return LPGEMM_ERR_INVALID_ARG;
        e_gemm.out = ws;
    }
    void *args[] = {(void *)&a,       (void *)&b,       (void *)&e_gemm, (void *)&m,
                    (void *)&n,       (void *)&k,       (void *)&tiles_m, (void *)&tiles_n,
                    (void *)&xcds,    (void *)&kc};
    hipError_t e = hipLaunchKernel(TK::template fn<OUT, SPLIT>(), dim3((unsigned)p.workgroups),
                                   dim3(TK::Cfg::kThreads), args, TK::Cfg::LDS_BYTES, stream);
    if (SPLIT && e == hipSuccess) {  // the slices hold partial sums only if the GEMM went out
        const int blocks = (int)std::min<int64_t>(ceil_div(count % 4 ? count : count / 4, 256), 4096);
        hipLaunchKernelGGL(sum_slices_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const int32_t *>(ws), static_cast<int32_t *>(epi.out), count,
                           p.k_chunks);
        e = hipGetLastError();
    }
    return e == hipSuccess ? LPGEMM_OK : LPGEMM_ERR_HIP;
}

// Launch the narrow-M kernel for K ranges up to KSTEPS * 1024 (SPLIT: several
// ranges added into C, which is zeroed first by a fill kernel); the first
// launch on each device raises its dynamic-LDS limit to the two strip buffers.
template <int VAR, int KSTEPS, int OUT, bool SPLIT, bool WHOLE_A = false>
lpgemm_status launch_skinny(const Plan &p, const uint8_t *a, const uint8_t *b, Epilogue epi, int m,
                            int n, int k, hipStream_t stream)
{
    using Cfg = SkinnyCfg<kSkinnyKW, KSTEPS>;
    constexpr auto kernel = &gemm_skinny_kernel<VAR, kSkinnyKW, KSTEPS, OUT, SPLIT, WHOLE_A>;
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        attr_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLdsBytes);
    });
    if (attr_err[dev] != hipSuccess) return LPGEMM_ERR_HIP;
    if (SPLIT) {
        const int64_t count = (int64_t)m * n;
        const int blocks = (int)std::min<int64_t>(ceil_div(count, 256), 65536);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<int32_t *>(epi.out), count);
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)p.workgroups), dim3(p.threads), Cfg::kLdsBytes, stream,
                       a, b, epi, m, n, k, p.kc);
    return launched();
}

// The narrow-M kernel taking every K range of its strips (no fill, no atomics).
template <int VAR, int OUT>
lpgemm_status launch_skinny_seq(const Plan &p, const uint8_t *a, const uint8_t *b, Epilogue epi,
                                int m, int n, int k, hipStream_t stream)
{
    using Cfg = SkinnyCfg<kSkinnyKW, 4>;
    constexpr auto kernel = &gemm_skinny_seq_kernel<VAR, kSkinnyKW, OUT>;
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        attr_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLdsBytes);
    });
    if (attr_err[dev] != hipSuccess) return LPGEMM_ERR_HIP;
    hipLaunchKernelGGL(kernel, dim3((unsigned)p.workgroups), dim3(p.threads), Cfg::kLdsBytes, stream,
                       a, b, epi, m, n, k, p.kc);
    return launched();
}

// The narrow-M instance for the plan's steps per wave and K ranges.
template <int VAR, int OUT>
lpgemm_status launch_skinny_steps(const Plan &p, const uint8_t *a, const uint8_t *b, Epilogue epi,
                                  int m, int n, int k, hipStream_t stream)
{
    if (p.k_chunks > 1 && p.k_steps != 4) return LPGEMM_ERR_INVALID_ARG;  // ranges > 4096 k
    if (p.k_chunks > 1 && p.k_seq) return launch_skinny_seq<VAR, OUT>(p, a, b, epi, m, n, k, stream);
    // int8 A over more than 8 rows: whole-line A loads (gemm_skinny.hpp)
    if constexpr (VAR == W4A8) {
        if (m > 8) {
            if constexpr (OUT == OUT_I32) {
                if (p.k_chunks > 1) return launch_skinny<VAR, 4, OUT, true, true>(p, a, b, epi, m, n, k, stream);
            } else {
                if (p.k_chunks > 1) return LPGEMM_ERR_INVALID_ARG;
            }
            switch (p.k_steps) {
            case 1: return launch_skinny<VAR, 1, OUT, false, true>(p, a, b, epi, m, n, k, stream);
            case 2: return launch_skinny<VAR, 2, OUT, false, true>(p, a, b, epi, m, n, k, stream);
            default: return launch_skinny<VAR, 4, OUT, false, true>(p, a, b, epi, m, n, k, stream);
            }
        }
    }
    if constexpr (OUT == OUT_I32) {
        if (p.k_chunks > 1) return launch_skinny<VAR, 4, OUT, true>(p, a, b, epi, m, n, k, stream);
    } else {
        if (p.k_chunks > 1) return LPGEMM_ERR_INVALID_ARG;
    }
    switch (p.k_steps) {
    case 1: return launch_skinny<VAR, 1, OUT, false>(p, a, b, epi, m, n, k, stream);
    case 2: return launch_skinny<VAR, 2, OUT, false>(p, a, b, epi, m, n, k, stream);
    default: return launch_skinny<VAR, 4, OUT, false>(p, a, b, epi, m, n, k, stream);
    }
}


// int4 x int4 on the FP6 matrix cores: re-encode A and B into the caller's
// workspace `ws` (the plan's ws_bytes), then multiply -- all on `stream`.
template <int OUT>
lpgemm_status launch_fp6(const Plan &p, const uint8_t *a, const uint8_t *b, Epilogue epi, int m,
                         int n, int k, void *ws, hipStream_t stream)
{
    constexpr auto kernel = &gemm_fp6_kernel<kFp6FM, kFp6FN, kFp6WM, kFp6WN, kFp6KS, kFp6Stages, OUT>;
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        attr_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            Fp6Tile::LDS_BYTES);
    });
    if (attr_err[dev] != hipSuccess) return LPGEMM_ERR_HIP;

    if (ws == nullptr) return LPGEMM_ERR_INVALID_ARG;
    const int64_t bytes_a = (int64_t)align_ws((uint64_t)fp6_bytes(m, k));
    uint8_t *a6 = static_cast<uint8_t *>(ws);
    uint8_t *b6 = a6 + bytes_a;
    const int64_t kgroups = ceil_div(ceil_div(k, 64), kFp6ConvWaves);
    const int64_t ga = ceil_div(m, 32) * kgroups, gb = ceil_div(n, 32) * kgroups;  // < 2^31 (plan)
    hipLaunchKernelGGL(fp6_convert_pair_kernel, dim3((unsigned)(ga + gb)), dim3(64 * kFp6ConvWaves), 0, stream, a, a6,
                       (int64_t)m, b, b6, (int64_t)n, k, ga);
    const uint8_t *ca6 = a6, *cb6 = b6;
    int tiles_m = p.tiles_m, tiles_n = p.tiles_n, xcds = kXcds;
    void *args[] = {(void *)&ca6, (void *)&cb6, (void *)&epi, (void *)&m,       (void *)&n,
                    (void *)&k,   (void *)&tiles_m, (void *)&tiles_n, (void *)&xcds};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel),
                                         dim3((unsigned)p.workgroups), dim3(Fp6Tile::kThreads),
                                         args, Fp6Tile::LDS_BYTES, stream);
    return (e == hipSuccess && hipGetLastError() == hipSuccess) ? LPGEMM_OK : LPGEMM_ERR_HIP;
}

// Launch the planned kernel for output format OUT.
template <int OUT>
lpgemm_status launch_gemm(const Plan &p, lpgemm_variant variant, const void *A, const void *B,
                          Epilogue epi, int64_t M, int64_t N, int64_t K, void *ws,
                          hipStream_t stream)
{
    const uint8_t *a = static_cast<const uint8_t *>(A);
    const uint8_t *b = static_cast<const uint8_t *>(B);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (p.kernel) {
    case LPGEMM_KERNEL_GENERAL: {
        const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16));
        if (variant == LPGEMM_VARIANT_I4I4)
            hipLaunchKernelGGL((gemm_general_kernel<I4I4, OUT>), grid, dim3(256), 0, stream, a, b, epi, M, N, K);
        else
            hipLaunchKernelGGL((gemm_general_kernel<W4A8, OUT>), grid, dim3(256), 0, stream, a, b, epi, M, N, K);
        return launched();
    }
    case LPGEMM_KERNEL_TILED:
        if constexpr (OUT == OUT_I32) {
            if (p.k_chunks > 1) {  // K ranges on 64- or 128-tiles
                if (p.tile == 128)
                    return variant == LPGEMM_VARIANT_I4I4
                               ? launch_tiled<I4Small, OUT, true>(p, a, b, epi, m, n, k, ws, stream)
                               : launch_tiled<W8Small, OUT, true>(p, a, b, epi, m, n, k, ws, stream);
                if (p.tile != 64) return LPGEMM_ERR_INVALID_ARG;
                return variant == LPGEMM_VARIANT_I4I4
                           ? launch_tiled<I4Tiny, OUT, true>(p, a, b, epi, m, n, k, ws, stream)
                           : launch_tiled<W8Tiny, OUT, true>(p, a, b, epi, m, n, k, ws, stream);
            }
        }
        if (variant == LPGEMM_VARIANT_I4I4)
            return p.tile == 256 ? launch_tiled<I4Large, OUT>(p, a, b, epi, m, n, k, ws, stream)
                   : p.tile == 128 ? launch_tiled<I4Small, OUT>(p, a, b, epi, m, n, k, ws, stream)
                                   : launch_tiled<I4Tiny, OUT>(p, a, b, epi, m, n, k, ws, stream);
        return p.tile == 256 ? launch_tiled<W8Large, OUT>(p, a, b, epi, m, n, k, ws, stream)
               : p.tile == 128 ? launch_tiled<W8Small, OUT>(p, a, b, epi, m, n, k, ws, stream)
                               : launch_tiled<W8Tiny, OUT>(p, a, b, epi, m, n, k, ws, stream);
    case LPGEMM_KERNEL_FP6:
        return launch_fp6<OUT>(p, a, b, epi, m, n, k, ws, stream);
    case LPGEMM_KERNEL_SKINNY:
        return variant == LPGEMM_VARIANT_I4I4
                   ? launch_skinny_steps<I4I4, OUT>(p, a, b, epi, m, n, k, stream)
                   : launch_skinny_steps<W4A8, OUT>(p, a, b, epi, m, n, k, stream);
    default:
        return LPGEMM_ERR_INVALID_ARG;
    }
}

// Workspace arguments: none (nullptr, 0), or device memory aligned to kWsAlign.
lpgemm_status check_workspace(const void *ws, size_t ws_bytes)
{
    if (ws_bytes == 0) return LPGEMM_OK;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1))) return LPGEMM_ERR_INVALID_ARG;
    return LPGEMM_OK;
}

// out_format: OUT_I32 for the plain entry points; scale pointers are used by
// the scaled formats only.  ws / ws_bytes: the caller's workspace (nullptr and
// 0 for the entry points without one).
lpgemm_status run_gemm(lpgemm_variant variant, const void *A, const void *B, void *C,
                       const float *scale_a, const float *scale_b, int out_format, int64_t M,
                       int64_t N, int64_t K, void *ws, size_t ws_bytes, hipStream_t stream)
{
    lpgemm_status st = check_args(A, B, C, M, N, K);
    if (st == LPGEMM_OK) st = check_workspace(ws, ws_bytes);
    if (st != LPGEMM_OK || M == 0 || N == 0) return st;
    if (out_format != OUT_I32) {
        if (scale_a == nullptr || scale_b == nullptr) return LPGEMM_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(scale_a) | reinterpret_cast<uintptr_t>(scale_b)) & 3u)
            return LPGEMM_ERR_INVALID_ARG;
        const uintptr_t elem = out_format == OUT_F32 ? 4u : 2u;
        if (reinterpret_cast<uintptr_t>(C) & (elem - 1)) return LPGEMM_ERR_INVALID_ARG;
    }
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    const Epilogue epi{C, scale_a, scale_b};
    if (K == 0) {
        if (out_format == OUT_I32) {
            const int64_t count = M * N;
            const int blocks = (int)std::min<int64_t>(ceil_div(count, 256), 65536);
            hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream,
                               static_cast<int32_t *>(C), count);
            return launched();
        }
        // The empty sum, scaled: the general kernel with no K loop.
        if (ceil_div(M, 16) > 65535 || ceil_div(N, 16) > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        Plan p;
        p.kernel = LPGEMM_KERNEL_GENERAL;
        switch (out_format) {
        case OUT_F32: return launch_gemm<OUT_F32>(p, variant, A, B, epi, M, N, K, nullptr, stream);
        case OUT_BF16: return launch_gemm<OUT_BF16>(p, variant, A, B, epi, M, N, K, nullptr, stream);
        default: return launch_gemm<OUT_F16>(p, variant, A, B, epi, M, N, K, nullptr, stream);
        }
    }
    Plan p;
    st = make_plan(variant, A, B, C, M, N, K, device_cu_count(), (lpgemm_kernel)t_override,
                   out_format == OUT_I32, ws_bytes, &p);
    if (st != LPGEMM_OK) return st;
    switch (out_format) {
    case OUT_I32: return launch_gemm<OUT_I32>(p, variant, A, B, epi, M, N, K, ws, stream);
    case OUT_F32: return launch_gemm<OUT_F32>(p, variant, A, B, epi, M, N, K, ws, stream);
    case OUT_BF16: return launch_gemm<OUT_BF16>(p, variant, A, B, epi, M, N, K, ws, stream);
    default: return launch_gemm<OUT_F16>(p, variant, A, B, epi, M, N, K, ws, stream);
    }
}

// fp8 product (VAR: FP8 or BF8): its own argument rules (no packing, any K),
// the tiled kernel when the operands allow 16-byte staging, else the general
// kernel.
template <int VAR, int OUT>
lpgemm_status launch_fp8(const uint8_t *A, const uint8_t *B, void *C, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream)
{
    const Epilogue epi{C, nullptr, nullptr};
    const uintptr_t c_align = OUT == OUT_F32 ? 16u : 4u;
    const bool fast = K > 0 && K % 16 == 0 && aligned16(A) && aligned16(B) &&
                      (reinterpret_cast<uintptr_t>(C) & (c_align - 1)) == 0;
    const int forced = t_override;
    if (forced == LPGEMM_KERNEL_SKINNY || forced == LPGEMM_KERNEL_FP6) return LPGEMM_ERR_UNSUPPORTED;
    const bool tiled_forced = forced == LPGEMM_KERNEL_TILED || forced == LPGEMM_KERNEL_TILED_128 ||
                              forced == LPGEMM_KERNEL_TILED_256 || forced == LPGEMM_KERNEL_TILED_64;
    if (tiled_forced && !fast) return LPGEMM_ERR_UNSUPPORTED;
    if (!fast || forced == LPGEMM_KERNEL_GENERAL) {
        if (ceil_div(M, 16) > 65535 || ceil_div(N, 16) > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16));
        hipLaunchKernelGGL((gemm_fp8_general_kernel<VAR, OUT>), grid, dim3(256), 0, stream, A, B, epi, M, N, K);
        return launched();
    }
    const int cu = device_cu_count();
    Plan p;
    const int64_t large_tiles = ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t small_tiles = ceil_div(M, 128) * ceil_div(N, 128);
    // As for the integer formats, except that the fp8 64-tiles (128 k per
    // stage) lose to 128-tiles covering half the compute units; up to kSmallM
    // rows never 256-tiles (64 x 65536 x 4096: 71.9 us on 256-tiles, 57.8 us
    // on 128-tiles).
    p.tile = forced == LPGEMM_KERNEL_TILED_256   ? 256
             : forced == LPGEMM_KERNEL_TILED_128 ? 128
             : forced == LPGEMM_KERNEL_TILED_64  ? 64
             : M > kSmallM && large_tiles * 4 >= (int64_t)cu * 3 ? 256
             : small_tiles * 2 >= (int64_t)cu     ? 128
                                                  : 64;
    p.tiles_m = (int)ceil_div(M, p.tile);
    p.tiles_n = (int)ceil_div(N, p.tile);
    p.workgroups = (int64_t)p.tiles_m * p.tiles_n;
    if (p.workgroups > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
    if (p.tile == 256) p.workgroups = std::min<int64_t>(p.workgroups, cu);
    const int m = (int)M, n = (int)N, k = (int)K;
    return p.tile == 256 ? launch_tiled<F8Large<VAR>, OUT>(p, A, B, epi, m, n, k, nullptr, stream)
           : p.tile == 128 ? launch_tiled<F8Small<VAR>, OUT>(p, A, B, epi, m, n, k, nullptr, stream)
                           : launch_tiled<F8Tiny<VAR>, OUT>(p, A, B, epi, m, n, k, nullptr, stream);
}

// VAR: FP8 (e4m3 operands, F32 or FP8_E4M3 output) or BF8 (e5m2 operands,
// F32 or FP8_E5M2 output).
template <int VAR>
lpgemm_status run_fp8(const uint8_t *A, const uint8_t *B, void *C, lpgemm_out_dtype out_dtype,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const lpgemm_out_dtype own = VAR == BF8 ? LPGEMM_OUT_FP8_E5M2 : LPGEMM_OUT_FP8_E4M3;
    if (M < 0 || N < 0 || K < 0) return LPGEMM_ERR_INVALID_ARG;
    if (out_dtype != LPGEMM_OUT_F32 && out_dtype != own) return LPGEMM_ERR_INVALID_ARG;
    if (K > LPGEMM_MAX_K) return LPGEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return LPGEMM_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return LPGEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    constexpr int OWN = VAR == BF8 ? OUT_E5M2 : OUT_E4M3;
    return out_dtype == LPGEMM_OUT_F32 ? launch_fp8<VAR, OUT_F32>(A, B, C, M, N, K, stream)
                                       : launch_fp8<VAR, OWN>(A, B, C, M, N, K, stream);
}

// lpgemm_out_dtype -> OutFormat; -1 for an unknown value.
int out_format_of(lpgemm_out_dtype d)
{
    switch (d) {
    case LPGEMM_OUT_F32: return OUT_F32;
    case LPGEMM_OUT_BF16: return OUT_BF16;
    case LPGEMM_OUT_F16: return OUT_F16;
    case LPGEMM_OUT_FP8_E4M3:
    case LPGEMM_OUT_FP8_E5M2: return -1;  // fp8 entry points only
    }
    return -1;
}

// ---- per-K-block scaled product ----------------------------------------------
// The tiled kernel with block scales (gemm_pipelined.hpp, SBP blocks per
// 128-k stage): 128 x 128 tiles (8 waves of 64 x 32: the fp32 accumulators
// beside the int32 ones fit two waves per SIMD without spilling, which 4
// waves of 64 x 64 do not) or 64 x 64 tiles (4 waves of 32 x 32), three
// stages, one tile per workgroup.
template <int VAR, int FM, int FN, int WM, int WN, int SBP>
struct BsKernel {
    using Cfg = PipeCfg<VAR, FM, FN, WM, WN, 128, 3, SBP>;
    template <int OUT>
    static void *fn()
    {
        return reinterpret_cast<void *>(&gemm_pipelined_kernel<VAR, FM, FN, WM, WN, 128, 3, OUT, false, SBP>);
    }
};

template <class TK, int OUT>
lpgemm_status launch_bs(int tiles_m, int tiles_n, const uint8_t *a, const uint8_t *b, Epilogue epi,
                        int m, int n, int k, hipStream_t stream)
{
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERR_HIP;
    std::call_once(once[dev], [dev] {
        attr_err[dev] = hipFuncSetAttribute(TK::template fn<OUT>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                                            TK::Cfg::LDS_BYTES_ALL);
    });
    if (attr_err[dev] != hipSuccess) return LPGEMM_ERR_HIP;
    int xcds = kXcds, kc = k;
    void *args[] = {(void *)&a,       (void *)&b,       (void *)&epi,  (void *)&m,    (void *)&n,
                    (void *)&k,       (void *)&tiles_m, (void *)&tiles_n, (void *)&xcds, (void *)&kc};
    const hipError_t e = hipLaunchKernel(TK::template fn<OUT>(), dim3((unsigned)(tiles_m * tiles_n)),
                                         dim3(TK::Cfg::kThreads), args, TK::Cfg::LDS_BYTES_ALL, stream);
    return e == hipSuccess ? LPGEMM_OK : LPGEMM_ERR_HIP;
}

template <int VAR, int OUT, int SBP>
lpgemm_status launch_bs_tile(int tile, int tiles_m, int tiles_n, const uint8_t *a, const uint8_t *b,
                             Epilogue epi, int m, int n, int k, hipStream_t stream)
{
    if (tile == 64)
        return launch_bs<BsKernel<VAR, 1, 1, 2, 2, SBP>, OUT>(tiles_m, tiles_n, a, b, epi, m, n, k, stream);
    if constexpr (SBP == 4)
        return launch_bs<BsKernel<VAR, 2, 1, 2, 4, SBP>, OUT>(tiles_m, tiles_n, a, b, epi, m, n, k, stream);
    else
        return launch_bs<BsKernel<VAR, 2, 2, 2, 2, SBP>, OUT>(tiles_m, tiles_n, a, b, epi, m, n, k, stream);
}

template <int VAR, int OUT>
lpgemm_status launch_blockscaled(const uint8_t *A, const uint8_t *B, Epilogue epi, int64_t M,
                                 int64_t N, int64_t K, hipStream_t stream)
{
    const uintptr_t d_align = OUT == OUT_F32 ? 16u : 8u;
    const bool fast = K > 0 && K % 32 == 0 && aligned16(A) && aligned16(B) &&
                      (reinterpret_cast<uintptr_t>(epi.out) & (d_align - 1)) == 0;
    const int forced = t_override;
    const bool t128 = forced == LPGEMM_KERNEL_TILED_128, t64 = forced == LPGEMM_KERNEL_TILED_64;
    if (forced != LPGEMM_KERNEL_AUTO && forced != LPGEMM_KERNEL_TILED && forced != LPGEMM_KERNEL_GENERAL &&
        !t128 && !t64)
        return LPGEMM_ERR_UNSUPPORTED;
    if ((forced == LPGEMM_KERNEL_TILED || t128 || t64) && !fast) return LPGEMM_ERR_UNSUPPORTED;
    if (!fast || forced == LPGEMM_KERNEL_GENERAL) {
        if (ceil_div(M, 16) > 65535 || ceil_div(N, 16) > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
        const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16));
        hipLaunchKernelGGL((gemm_blockscaled_general_kernel<VAR, OUT>), grid, dim3(256), 0, stream, A, B, epi,
                           M, N, K);
        return launched();
    }
    // 64-tiles for up to 64 rows (16 x 28672 x 8192, g = 128: 67 against 80 us)
    // and where 128-tiles would leave more than half the compute units idle;
    // else 128-tiles (4096^3 W4A8, g = 128: 188 against 238 us)
    const int64_t small_tiles = ceil_div(M, 128) * ceil_div(N, 128);
    const int tile = t128 ? 128
                     : t64 ? 64
                     : M > 64 && small_tiles * 2 >= (int64_t)device_cu_count() ? 128
                                                                                  : 64;
    const int64_t tiles_m = ceil_div(M, tile), tiles_n = ceil_div(N, tile);
    if (tiles_m * tiles_n > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
    const int m = (int)M, n = (int)N, k = (int)K, tm = (int)tiles_m, tn = (int)tiles_n;
    switch (epi.lg) {
    case 5: return launch_bs_tile<VAR, OUT, 4>(tile, tm, tn, A, B, epi, m, n, k, stream);
    case 6: return launch_bs_tile<VAR, OUT, 2>(tile, tm, tn, A, B, epi, m, n, k, stream);
    default: return launch_bs_tile<VAR, OUT, 1>(tile, tm, tn, A, B, epi, m, n, k, stream);
    }
}

// Arguments of the block-scaled entry points; then the launch.
template <int VAR>
lpgemm_status run_blockscaled(const void *A, const uint8_t *B, const float *SFA, const float *SFB,
                              int64_t g, void *D, lpgemm_out_dtype out_dtype, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 0 || (K & 1)) return LPGEMM_ERR_INVALID_ARG;
    if (g < 32 || g > ((int64_t)1 << 30) || (g & (g - 1))) return LPGEMM_ERR_INVALID_ARG;
    const int f = out_format_of(out_dtype);
    if (f < 0) return LPGEMM_ERR_INVALID_ARG;
    if (K > LPGEMM_MAX_K) return LPGEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return LPGEMM_OK;
    const uintptr_t d_elt = f == OUT_F32 ? 4u : 2u;
    if (D == nullptr || (reinterpret_cast<uintptr_t>(D) & (d_elt - 1))) return LPGEMM_ERR_INVALID_ARG;
    if (K > 0 && (A == nullptr || B == nullptr || SFA == nullptr || SFB == nullptr ||
                  (reinterpret_cast<uintptr_t>(SFA) & 3u) || (reinterpret_cast<uintptr_t>(SFB) & 3u)))
        return LPGEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERR_UNSUPPORTED;
    int lg = 0;
    while (((int64_t)1 << lg) < g) ++lg;
    Epilogue epi{D, SFA, SFB};
    epi.nb = (int32_t)ceil_div(K, g);
    epi.lg = lg;
    const uint8_t *a = static_cast<const uint8_t *>(A);
    (void)hipGetLastError();
    switch (f) {
    case OUT_F32: return launch_blockscaled<VAR, OUT_F32>(a, B, epi, M, N, K, stream);
    case OUT_BF16: return launch_blockscaled<VAR, OUT_BF16>(a, B, epi, M, N, K, stream);
    default: return launch_blockscaled<VAR, OUT_F16>(a, B, epi, M, N, K, stream);
    }
}

lpgemm_status run_elementwise(bool pack, const void *src, void *dst, int64_t rows, int64_t K,
                              hipStream_t stream)
{
    if (rows < 0 || K < 0 || (K & 1)) return LPGEMM_ERR_INVALID_ARG;
    if (K > 0 && rows > INT64_MAX / (K / 2)) return LPGEMM_ERR_UNSUPPORTED;  // bytes would overflow
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
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, nullptr, nullptr, OUT_I32, M, N, K,
                    nullptr, 0, stream);
}

lpgemm_status lpgemm_w4a8(const int8_t *A, const uint8_t *B_packed, int32_t *C, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream)
{
    return run_gemm(LPGEMM_VARIANT_W4A8, A, B_packed, C, nullptr, nullptr, OUT_I32, M, N, K,
                    nullptr, 0, stream);
}

lpgemm_status lpgemm_int4_int4_ws(const void *A_packed, const void *B_packed, int32_t *C, int64_t M,
                                  int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream)
{
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, nullptr, nullptr, OUT_I32, M, N, K,
                    workspace, workspace_bytes, stream);
}

lpgemm_status lpgemm_int4_int4_noalloc(const void *A_packed, const void *B_packed, int32_t *C,
                                       int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    lpgemm_status st = check_args(A_packed, B_packed, C, M, N, K);
    if (st != LPGEMM_OK || M == 0 || N == 0 || K == 0)
        return st != LPGEMM_OK ? st
                               : run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, nullptr,
                                          nullptr, OUT_I32, M, N, K, nullptr, 0, stream);
    // the scratch the call would use with unlimited workspace
    Plan p;
    st = make_plan(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, M, N, K, device_cu_count(),
                   (lpgemm_kernel)t_override, true, UINT64_MAX, &p);
    if (st != LPGEMM_OK) return st;
    if ((uint64_t)p.ws_bytes > LPGEMM_STATIC_SCRATCH_BYTES) return LPGEMM_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        st = static_scratch(&ws);
        if (st != LPGEMM_OK) return st;
    }
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, C, nullptr, nullptr, OUT_I32, M, N, K,
                    ws, ws ? (size_t)LPGEMM_STATIC_SCRATCH_BYTES : 0, stream);
}

lpgemm_status lpgemm_w4a8_ws(const int8_t *A, const uint8_t *B_packed, int32_t *C, int64_t M,
                             int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    return run_gemm(LPGEMM_VARIANT_W4A8, A, B_packed, C, nullptr, nullptr, OUT_I32, M, N, K,
                    workspace, workspace_bytes, stream);
}

lpgemm_status lpgemm_int4_int4_scaled(const void *A_packed, const void *B_packed,
                                      const float *scale_a, const float *scale_b, void *D,
                                      lpgemm_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                      hipStream_t stream)
{
    const int f = out_format_of(out_dtype);
    if (f < 0) return LPGEMM_ERR_INVALID_ARG;
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, D, scale_a, scale_b, f, M, N, K,
                    nullptr, 0, stream);
}

lpgemm_status lpgemm_int4_int4_scaled_ws(const void *A_packed, const void *B_packed,
                                         const float *scale_a, const float *scale_b, void *D,
                                         lpgemm_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int f = out_format_of(out_dtype);
    if (f < 0) return LPGEMM_ERR_INVALID_ARG;
    return run_gemm(LPGEMM_VARIANT_I4I4, A_packed, B_packed, D, scale_a, scale_b, f, M, N, K,
                    workspace, workspace_bytes, stream);
}

lpgemm_status lpgemm_w4a8_scaled(const int8_t *A, const uint8_t *B_packed, const float *scale_a,
                                 const float *scale_b, void *D, lpgemm_out_dtype out_dtype,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int f = out_format_of(out_dtype);
    if (f < 0) return LPGEMM_ERR_INVALID_ARG;
    return run_gemm(LPGEMM_VARIANT_W4A8, A, B_packed, D, scale_a, scale_b, f, M, N, K, nullptr, 0,
                    stream);
}

lpgemm_status lpgemm_int4_int4_blockscaled(const void *A_packed, const void *B_packed, const float *SFA,
                                           const float *SFB, int64_t g, void *D,
                                           lpgemm_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                           hipStream_t stream)
{
    return run_blockscaled<I4I4>(A_packed, static_cast<const uint8_t *>(B_packed), SFA, SFB, g, D, out_dtype,
                                 M, N, K, stream);
}

lpgemm_status lpgemm_w4a8_blockscaled(const int8_t *A, const uint8_t *B_packed, const float *SFA,
                                      const float *SFB, int64_t g, void *D, lpgemm_out_dtype out_dtype,
                                      int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    return run_blockscaled<W4A8>(A, B_packed, SFA, SFB, g, D, out_dtype, M, N, K, stream);
}

lpgemm_status lpgemm_fp8_e4m3(const uint8_t *A, const uint8_t *B, void *C,
                              lpgemm_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream)
{
    return run_fp8<FP8>(A, B, C, out_dtype, M, N, K, stream);
}

lpgemm_status lpgemm_fp8_e5m2(const uint8_t *A, const uint8_t *B, void *C,
                              lpgemm_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream)
{
    return run_fp8<BF8>(A, B, C, out_dtype, M, N, K, stream);
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
    case LPGEMM_ERR_SCRATCH_LIMIT: return "needs more scratch than the library's static scratch holds";
    }
    return "unknown status";
}

lpgemm_status lpgemm_plan(lpgemm_variant variant, const void *A, const void *B, const void *C,
                          int64_t M, int64_t N, int64_t K, size_t workspace_bytes,
                          int32_t cu_count, lpgemm_plan_info *info)
{
    if (info == nullptr || (variant != LPGEMM_VARIANT_I4I4 && variant != LPGEMM_VARIANT_W4A8))
        return LPGEMM_ERR_INVALID_ARG;
    lpgemm_status st = check_args(A, B, C, M, N, K);
    if (st != LPGEMM_OK) return st;
    *info = lpgemm_plan_info{};
    if (M == 0 || N == 0 || K == 0) return LPGEMM_OK;  // nothing, or a zero fill
    Plan p;
    st = make_plan(variant, A, B, C, M, N, K, cu_count > 0 ? cu_count : kDefaultCUs,
                   (lpgemm_kernel)t_override, true, workspace_bytes, &p);
    if (st != LPGEMM_OK) return st;
    info->kernel = p.kernel;
    info->tile_m = p.tile_m;
    info->tile_n = p.tile_n;
    info->k_split = p.k_split;
    info->workgroups = p.workgroups;
    info->threads = p.threads;
    info->k_chunks = p.k_chunks;
    info->workspace_bytes = p.ws_bytes;
    return LPGEMM_OK;
}

lpgemm_status lpgemm_workspace_size(lpgemm_variant variant, int32_t scaled, int64_t M, int64_t N,
                                    int64_t K, int32_t cu_count, size_t *bytes)
{
    if (bytes == nullptr || (variant != LPGEMM_VARIANT_I4I4 && variant != LPGEMM_VARIANT_W4A8) ||
        (scaled != 0 && scaled != 1))
        return LPGEMM_ERR_INVALID_ARG;
    *bytes = 0;
    // any 256-byte aligned addresses: the fast kernels' conditions on them hold
    const void *dev = reinterpret_cast<const void *>(uintptr_t{256});
    lpgemm_status st = check_args(dev, dev, dev, M, N, K);
    if (st != LPGEMM_OK || M == 0 || N == 0 || K == 0) return st;
    Plan p;
    st = make_plan(variant, dev, dev, dev, M, N, K, cu_count > 0 ? cu_count : kDefaultCUs,
                   LPGEMM_KERNEL_AUTO, scaled == 0, UINT64_MAX, &p);
    if (st != LPGEMM_OK) return st;
    *bytes = (size_t)p.ws_bytes;
    return LPGEMM_OK;
}

lpgemm_status lpgemm_set_kernel_override(lpgemm_kernel kernel)
{
    if (kernel < LPGEMM_KERNEL_AUTO || kernel > LPGEMM_KERNEL_FP6) return LPGEMM_ERR_INVALID_ARG;
    t_override = kernel;
    return LPGEMM_OK;
}

}  // extern "C"
