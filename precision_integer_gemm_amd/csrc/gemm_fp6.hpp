// gemm_fp6.hpp -- int4 x int4 through gfx950's FP6 matrix cores.
//
// CDNA4's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 6-bit floating-point
// operands at twice the int8 rate.  Every int4 value v in [-8, 7] is exact in
// FP6 E3M2 (sign, 3 exponent bits with bias 3, 2 mantissa bits): |v| needs at
// most three significant bits and 8 = 1.00b x 2^3 is the largest magnitude.
// Each product is an integer of magnitude <= 64.  The matrix cores do not add
// in IEEE binary32; measured on MI355X, an instruction sums its products in
// groups of 8 consecutive k on a grid of 2^-14 of the group's largest product
// (lower bits truncated) and combines the group sums with the accumulator in
// binary32, rounding to nearest even.  With integer products of at most 2^6
// the grid step is below 1, and every combined value is an integer of
// magnitude <= 64 * 131070 < 2^23, exact in binary32: the fp32 accumulator
// holds the exact integer dot product for K <= 131070, and converting it to
// int32 gives the same C as the int8 path.  Checked bit for bit against the
// oracle on the whole 8192^3 product, and on closed forms at K = 131040:
// all -8 operands, mixed signs, and a single odd product next to partial sums
// of 8386496 in the first, a middle or the last 64-k block.
//
// Two steps per call:
//  1. fp6_convert_pair_kernel re-encodes both packed int4 operands, in one
//     launch, into fragment-major FP6 arrays X6[rb][kb][1536 bytes]: row block rb (32
//     rows), k block kb (64 k).  Inside a fragment, lane slot l covers row
//     l % 32 and k = 64 kb + 32 (l / 32) + e for e = 0..31, 32 six-bit codes
//     with element e at bits 6e .. 6e+5 of a 192-bit value -- exactly the
//     operand one MFMA lane supplies.  The first 16 bytes of every slot sit at
//     16 l, the last 8 at 1024 + 8 l, so a wave reads a fragment from LDS with
//     one conflict-free ds_read_b128 and one ds_read_b64.  Rows past the
//     matrix and k past K encode zero.  The conversion itself is exact: each
//     nibble becomes an f16 integer (1024 + (v + 8) - 1032 in f16 arithmetic)
//     and v_cvt_scalef32_pk32_bf6_f16 turns 32 of them into E3M2 codes.
//  2. gemm_fp6_kernel: the persistent, XCD-aware tile loop of the int8 tiled
//     kernel, with each stage of A6 and B6 copied into LDS by direct-to-LDS
//     loads of whole 1 KB pieces (a row block's fragments for one stage are
//     contiguous in memory), then one MFMA per 32x32 block per 64 k.  The
//     copy that refills a stage's slot is issued after the MFMAs of the step
//     that follows the stage's barrier, so those MFMAs start first (with
//     three stages this measured 2-4% faster than issuing it at the barrier).
//     B is the MFMA's row operand and A its column operand, so each lane ends
//     with four consecutive n of one m (16-byte stores).
#pragma once

#include "device_common.hpp"

namespace lpgemm {

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x6 __attribute__((ext_vector_type(6)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x32 __attribute__((ext_vector_type(32)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFp6FragBytes = 1536;  // 64 lanes x 32 six-bit codes
constexpr int kFp6MfmaFormat = 3;    // E3M2 operand format of the f8f6f4 MFMA
constexpr int kFp6UnitScale = 127;   // E8M0 exponent of a scale of 1.0

// Bytes of the FP6 copy of an R x K int4 operand.
__host__ __device__ inline int64_t fp6_bytes(int64_t R, int64_t K)
{
    return ((R + 31) / 32) * ((K + 63) / 64) * kFp6FragBytes;
}

// 32 packed int4 values (16 bytes, element e in nibble e) -> 32 E3M2 codes.
__device__ __forceinline__ i32x6 e3m2_from_int4(i32x4 q)
{
    f16x32 h;
    const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t x = (uint32_t)q[j] ^ 0x88888888u;  // every nibble: v + 8 in 0..15
        const uint32_t even = x & 0x0F0F0F0Fu;
        const uint32_t odd = (x >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // f16 bit patterns 0x6400 | u encode 1024 + u exactly.
            const uint32_t p = ((even >> (8 * i)) & 0xFFu) | (((odd >> (8 * i)) & 0xFFu) << 16) |
                               0x64006400u;
            const f16x2 v = __builtin_bit_cast(f16x2, p) - bias;
            h[8 * j + 2 * i] = v.x;
            h[8 * j + 2 * i + 1] = v.y;
        }
    }
    return __builtin_amdgcn_cvt_scalef32_pk32_bf6_f16(h, 1.0f);
}

// Both operands in one launch, one thread per fragment lane slot.  A
// workgroup of kFp6ConvWaves waves takes one row block over that many
// consecutive k blocks (wave w: k block kFp6ConvWaves g + w), so each 32-row
// group's 512-byte run of packed input is read once, by the waves together;
// lane l of a wave loads the 16 bytes of its slot (row l % 32, k half l / 32),
// encodes them and writes the slot's 16 + 8 bytes (each wave writes one whole
// 1.5 KB fragment).  Workgroups [0, ga) cover A, the rest B.  Requires
// K % 32 == 0 and 16-byte aligned operands.  Measured on MI355X with both
// operands evicted from the caches first (outputs byte-identical): four waves
// per workgroup 32.6 us for 8192^3 and 16.4 us for 3000 x 5120 x 6144, eight
// 31.2 / 15.0 us, sixteen 30.4 / 15.4 us (5.5 TB/s of packed reads and FP6
// writes); two or four k blocks per wave were slower.  (The earlier two
// launches of a 32-row x 2048-k LDS-staged kernel: 8192^3 34.1 us warm.)
constexpr int kFp6ConvWaves = 16;
__global__ __launch_bounds__(64 * kFp6ConvWaves) void fp6_convert_pair_kernel(const uint8_t *__restrict__ A,
                                                               uint8_t *__restrict__ A6, int64_t MA,
                                                               const uint8_t *__restrict__ B,
                                                               uint8_t *__restrict__ B6, int64_t NB,
                                                               int K, int64_t ga)
{
    const int K64 = (K + 63) / 64;
    const int kgroups = (K64 + kFp6ConvWaves - 1) / kFp6ConvWaves;
    const bool is_a = (int64_t)blockIdx.x < ga;
    const int64_t g = is_a ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - ga;
    const uint8_t *X = is_a ? A : B;
    uint8_t *X6 = is_a ? A6 : B6;
    const int64_t R = is_a ? MA : NB;
    const int64_t rb = g / kgroups;
    const int kb = (int)(g % kgroups) * kFp6ConvWaves + (int)(threadIdx.x >> 6);
    if (kb >= K64) return;
    const int lane = threadIdx.x & 63;
    const int64_t row = rb * 32 + (lane & 31);
    const int64_t ldx = K / 2;
    const int64_t byte = (int64_t)kb * 32 + 16 * (lane >> 5);
    i32x4 q = {0, 0, 0, 0};
    if (row < R && byte < ldx) q = *reinterpret_cast<const i32x4 *>(X + row * ldx + byte);
    const i32x6 o = e3m2_from_int4(q);
    uint8_t *dst = X6 + (rb * K64 + kb) * kFp6FragBytes;
    *reinterpret_cast<i32x4 *>(dst + 16 * lane) = i32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<i32x2 *>(dst + 1024 + 8 * lane) = i32x2{o[4], o[5]};
}

template <int FM, int FN, int WM, int WN, int KS, int STAGES>
struct Fp6Cfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = WM * FM * 32;
    static constexpr int BN = WN * FN * 32;
    static constexpr int SPAN = KS * kFp6FragBytes;  // one row block's bytes per stage
    static constexpr int A_BYTES = (BM / 32) * SPAN;
    static constexpr int B_BYTES = (BN / 32) * SPAN;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Two slots for a tile's scale vectors (scaled outputs): BM + BN floats,
    // rounded up to whole 64-float DMA instructions.
    static constexpr int SCALE_SLOT = 4 * ((BM + BN + 63) / 64 * 64);
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + 2 * SCALE_SLOT;
    static constexpr int NA = A_BYTES / 1024 / kWaves;  // DMA instructions per wave per stage
    static constexpr int NB = B_BYTES / 1024 / kWaves;
    static_assert(NA * 1024 * kWaves == A_BYTES && NB * 1024 * kWaves == B_BYTES,
                  "each wave must issue whole 1 KB DMA instructions");
    static constexpr bool kFits = STAGES >= 2 && LDS_BYTES <= 160 * 1024;
};

// C[M,N] from the FP6 copies A6 (of A[M,K]) and B6 (of B[N,K]).  Requirements
// (checked on the host): K % 32 == 0, 0 < K <= 131070, M, N < 2^31.
template <int FM, int FN, int WM, int WN, int KS, int STAGES, int OUT>
__global__ __launch_bounds__(64 * WM * WN, (FM * FN <= 8) ? 2 : 1) void gemm_fp6_kernel(
    const uint8_t *__restrict__ A6, const uint8_t *__restrict__ B6, Epilogue epi, int M, int N,
    int K, int tiles_m, int tiles_n, int xcds)
{
    using Cfg = Fp6Cfg<FM, FN, WM, WN, KS, STAGES>;
    static_assert(Cfg::kFits, "LDS ring does not fit in 160 KB");
    constexpr int NA = Cfg::NA, NB = Cfg::NB, SPAN = Cfg::SPAN;
    constexpr int kPerStage = NA + NB;
    constexpr int kPrologue = STAGES;
    constexpr int kStores = FN * FM * 4;
    extern __shared__ __align__(1024) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int K64 = (K + 63) / 64;
    const int ktiles = (K64 + KS - 1) / KS;
    const int RBA = (M + 31) / 32, RBB = (N + 31) / 32;

    // Per-lane source of each DMA instruction: a stage holds, per row block,
    // KS consecutive fragments, contiguous in memory and in LDS.
    uint32_t a_off[NA], b_off[NB];
    int a_frag[NA], b_frag[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int byte = (wave * NA + i) * 1024 + 16 * lane;
        const int rb = byte / SPAN, within = byte % SPAN;
        a_frag[i] = within / kFp6FragBytes;
        a_off[i] = (uint32_t)rb * (uint32_t)K64 * kFp6FragBytes + (uint32_t)within;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int byte = (wave * NB + i) * 1024 + 16 * lane;
        const int rb = byte / SPAN, within = byte % SPAN;
        b_frag[i] = within / kFp6FragBytes;
        b_off[i] = (uint32_t)rb * (uint32_t)K64 * kFp6FragBytes + (uint32_t)within;
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    // Tile order as in the int8 tiled kernel: XCD-contiguous bands of 4 tile rows.
    const int nblocks = tiles_m * tiles_n;
    const int whole = nblocks - nblocks % xcds;
    auto tile_origin = [&](int v, int &m0, int &n0) {
        int id = v;
        if (id < whole) id = (id % xcds) * (whole / xcds) + id / xcds;
        constexpr int kBand = 4;
        const int band = id / (kBand * tiles_n);
        const int band_m0 = band * kBand;
        const int band_rows = min(kBand, tiles_m - band_m0);
        const int in_band = id - band * kBand * tiles_n;
        m0 = (band_m0 + in_band % band_rows) * Cfg::BM;
        n0 = (in_band / band_rows) * Cfg::BN;
    };

    int v = blockIdx.x;
    int m0, n0;
    tile_origin(v, m0, n0);
    // Buffer resources start at the tile's first row block, so offsets stay
    // below 2^31; row blocks past the matrix lie beyond the range: zeros.
    constexpr bool kScaled = OUT != OUT_I32;
    i32x4 rsrc_a, rsrc_b, rsrc_sa, rsrc_sb;
    auto set_rsrc = [&]() {
        if constexpr (kScaled) {
            rsrc_sa = make_rsrc(epi.scale_a + m0, (uint32_t)min(Cfg::BM, M - m0) * 4u);
            rsrc_sb = make_rsrc(epi.scale_b + n0, (uint32_t)min(Cfg::BN, N - n0) * 4u);
        }
        const int rba = m0 / 32, rbb = n0 / 32;
        rsrc_a = make_rsrc(A6 + (int64_t)rba * K64 * kFp6FragBytes,
                           (uint32_t)min(Cfg::BM / 32, RBA - rba) * (uint32_t)K64 * kFp6FragBytes);
        rsrc_b = make_rsrc(B6 + (int64_t)rbb * K64 * kFp6FragBytes,
                           (uint32_t)min(Cfg::BN / 32, RBB - rbb) * (uint32_t)K64 * kFp6FragBytes);
    };
    set_rsrc();

    // DMA of stage kt into its ring slot; fragments past the last k block
    // read out of range (zeros).
    auto issue_stage = [&](int kt) {
        const uint32_t base = lds0 + (uint32_t)(kt % STAGES) * Cfg::STAGE_BYTES;
        const int kb0 = kt * KS;
        const uint32_t koff = (uint32_t)kb0 * kFp6FragBytes;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const uint32_t off = (kb0 + a_frag[i] < K64) ? a_off[i] + koff : kOutOfRange;
            dma16(rsrc_a, off, base + (uint32_t)(wave * NA + i) * 1024u);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint32_t off = (kb0 + b_frag[i] < K64) ? b_off[i] + koff : kOutOfRange;
            dma16(rsrc_b, off, base + Cfg::A_BYTES + (uint32_t)(wave * NB + i) * 1024u);
        }
    };

    const int h = lane >> 5;
    const int r32 = lane & 31;

    struct Frags {
        i32x8 b[FN];
        i32x8 a[FM];
    };
    // The 8-byte half is read through a volatile LDS pointer: otherwise the
    // compiler pairs the halves of two fragments into one ds_read2st64_b64,
    // whose result then has to be moved into the two operands, and waits for
    // it right after issuing it.
    auto frag_at = [&](const uint8_t *p) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(p + 16 * lane);
        const i32x2 hi = *(const volatile __attribute__((address_space(3))) i32x2 *)(p + 1024 + 8 * lane);
        return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, 0, 0};  // the MFMA reads six dwords
    };
    auto read_frags = [&](int slot, int step, Frags &f) {
        const uint8_t *sa = smem + slot * Cfg::STAGE_BYTES;
        const uint8_t *sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) f.b[fn] = frag_at(sb + ((wn * FN + fn) * KS + step) * kFp6FragBytes);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) f.a[fm] = frag_at(sa + ((wm * FM + fm) * KS + step) * kFp6FragBytes);
    };

    f32x16 acc[FN][FM];
    auto compute = [&](const Frags &f) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[fn], f.a[fm], acc[fn][fm], kFp6MfmaFormat, kFp6MfmaFormat, 0, kFp6UnitScale,
                    0, kFp6UnitScale);
    };

    auto wait_tiles_after = [&](int after) {
        if (after >= 2)
            wait_vmcnt<2 * kPerStage>();
        else if (after == 1)
            wait_vmcnt<kPerStage>();
        else
            wait_vmcnt<0>();
    };

    // Scaled outputs: a tile's scale vectors go into LDS slot p with the
    // tile's first copies, element e = 64 wave + lane being scale_a[m0 + e]
    // for e < BM, then scale_b[n0 + e - BM] (zeros past M and N).  The
    // epilogue then reads them from LDS, so no global load of its own has to
    // be waited for behind the next tile's copies.
    const uint32_t lds_scales = lds0 + (uint32_t)(STAGES * Cfg::STAGE_BYTES);
    int par = 0;  // slot of the current tile's scales
    auto issue_scales = [&](int p) {
        if constexpr (kScaled) {
            static_assert(Cfg::BM % 64 == 0, "a scale DMA instruction must not straddle the two vectors");
            for (int e0 = wave * 64; e0 < Cfg::BM + Cfg::BN; e0 += 64 * Cfg::kWaves) {  // wave-uniform
                const bool isb = e0 >= Cfg::BM;
                const uint32_t off = (uint32_t)((isb ? e0 - Cfg::BM : e0) + lane) * 4u;
                dma4(isb ? rsrc_sb : rsrc_sa, off, lds_scales + (uint32_t)(p * Cfg::SCALE_SLOT + e0 * 4));
            }
        }
    };
    issue_scales(0);
#pragma unroll
    for (int s = 0; s < kPrologue; ++s) issue_stage(s);
    bool stores_pending = false;

    for (;;) {
        if (stores_pending)
            wait_vmcnt<(kPrologue - 1) * kPerStage + kStores>();
        else
            wait_vmcnt<(kPrologue - 1) * kPerStage>();
        lds_barrier();

#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};
        Frags cur, nxt;
        read_frags(0, 0, cur);

        for (int kt = 0; kt + 1 < ktiles; ++kt) {
            const int slot = kt % STAGES;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                if (st + 1 < KS) {
                    read_frags(slot, st + 1, nxt);
                } else {
                    wait_tiles_after(STAGES - 2);
                    lds_barrier();
                    read_frags((kt + 1) % STAGES, 0, nxt);
                }
                compute(cur);
                // The next step's fragment reads go out between this step's
                // first MFMAs (three after each of the first four), so their
                // latency hides behind the wave's own matrix-core work.
                constexpr int kReads = 2 * (FM + FN), kPer = 3;
                constexpr int kGroups = (kReads + kPer - 1) / kPer;
                static_assert(kGroups <= FM * FN, "more read groups than MFMAs");
#pragma unroll
                for (int g = 0; g + 1 < kGroups; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);  // LDS reads
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, kReads - (kGroups - 1) * kPer, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - kGroups, 0);
                // The slot of stage kt is free once every wave has passed the
                // barrier; its refill goes out after this step's MFMAs.
                if (st + 1 == KS) issue_stage(kt + STAGES);
                cur = nxt;
            }
        }
        {
            const int slot = (ktiles - 1) % STAGES;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                if (st + 1 < KS) read_frags(slot, st + 1, nxt);
                compute(cur);
                cur = nxt;
            }
        }
        wait_vmcnt<0>();

        const int tm0 = m0, tn0 = n0;
        const int tpar = par;
        const int vn = v + (int)gridDim.x;
        auto store_tile = [&]() {
            float sa[FM], sb[FN][4][4];
            if constexpr (kScaled) {
                const float *ss =
                    reinterpret_cast<const float *>(smem + STAGES * Cfg::STAGE_BYTES + tpar * Cfg::SCALE_SLOT);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) sa[fm] = ss[(wm * FM + fm) * 32 + r32];
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const f32x4 q = *reinterpret_cast<const f32x4 *>(
                            ss + Cfg::BM + (wn * FN + fn) * 32 + 8 * rg + 4 * h);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sb[fn][rg][i] = q[i];
                    }
            } else {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) sa[fm] = 0.f;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sb[fn][rg][i] = 0.f;
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int m = tm0 + (wm * FM + fm) * 32 + r32;
                    if (m >= M) continue;
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int n = tn0 + (wn * FN + fn) * 32 + 8 * rg + 4 * h;
                        // exact integers below 2^24: the conversion is exact
                        const i32x4 c = i32x4{(int32_t)acc[fn][fm][4 * rg + 0], (int32_t)acc[fn][fm][4 * rg + 1],
                                              (int32_t)acc[fn][fm][4 * rg + 2], (int32_t)acc[fn][fm][4 * rg + 3]};
                        store_row4<OUT>(epi, m, N, n, c, sa[fm], sb[fn][rg]);
                    }
                }
        };
        auto start_next = [&]() {
            lds_barrier();  // every wave is done reading this tile's slots
            if (vn < nblocks) {
                tile_origin(vn, m0, n0);
                set_rsrc();
                issue_scales(par ^ 1);
#pragma unroll
                for (int s = 0; s < kPrologue; ++s) issue_stage(s);
            }
        };
        // The workgroup's last tile: no copies follow, so the stage ring is
        // free and C goes out through it as whole rows, one 1 KB row piece
        // per wave instruction (the MFMA layout stores 32-byte pieces of 32
        // rows per instruction, which HBM absorbs more slowly).  Passes of
        // kRows rows: the waves holding a pass's 32-row blocks write them
        // (exact integers, padded rows), then every wave stores rows of it.
        constexpr bool kStageC = Cfg::BN == 256;
        auto store_tile_staged = [&]() {
          if constexpr (kStageC) {
            // Lane indices taken afresh here (an opaque copy of the thread
            // id), so that no address of this path is computed before the
            // K loop and kept live through it.
            int tid = (int)threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int sl = tid & 63, sr32 = sl & 31, sh = sl >> 5;
            constexpr int kPitch = Cfg::BN * 4 + 16;
            constexpr int kRows = ((STAGES * Cfg::STAGE_BYTES / kPitch) / 32 * 32) < Cfg::BM
                                      ? (STAGES * Cfg::STAGE_BYTES / kPitch) / 32 * 32
                                      : Cfg::BM;
            static_assert(kRows >= 32, "the stage ring holds fewer than 32 staged rows");
            const float *ss =
                reinterpret_cast<const float *>(smem + STAGES * Cfg::STAGE_BYTES + tpar * Cfg::SCALE_SLOT);
            float sb4[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kScaled) {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(ss + Cfg::BM + 4 * sl);
#pragma unroll
                for (int i = 0; i < 4; ++i) sb4[i] = q[i];
            }
#pragma unroll
            for (int p0 = 0; p0 < Cfg::BM; p0 += kRows) {
                if (p0 > 0) lds_barrier();  // the previous pass's rows have been read
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int rb = (wm * FM + fm) * 32;  // first tile row of the block
                    if (rb < p0 || rb >= p0 + kRows) continue;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) {
                            const int col = (wn * FN + fn) * 32 + 8 * rg + 4 * sh;
                            // exact integers below 2^24: the conversion is exact
                            const i32x4 c = i32x4{(int32_t)acc[fn][fm][4 * rg + 0], (int32_t)acc[fn][fm][4 * rg + 1],
                                                  (int32_t)acc[fn][fm][4 * rg + 2], (int32_t)acc[fn][fm][4 * rg + 3]};
                            *reinterpret_cast<i32x4 *>(smem + (rb - p0 + sr32) * kPitch + 4 * col) = c;
                        }
                }
                lds_barrier();
                for (int r = p0 + wave; r < p0 + kRows && r < Cfg::BM; r += Cfg::kWaves) {
                    const int m = tm0 + r;
                    if (m >= M) break;
                    const i32x4 c = *reinterpret_cast<const i32x4 *>(smem + (r - p0) * kPitch + 16 * sl);
                    store_row4<OUT>(epi, m, N, tn0 + 4 * sl, c, kScaled ? ss[r] : 0.f, sb4);
                }
            }
          }
        };
        // The next tile's copies go out before this tile's stores (one store
        // instruction per row segment of a whole tile, in every format), so
        // the next tile's first wait does not also wait for the stores.
        start_next();
        if constexpr (kStageC) {
            if (vn >= nblocks) {
                store_tile_staged();
                break;
            }
        }
        store_tile();
        if (vn >= nblocks) break;
        par ^= 1;
        stores_pending = (N % 4) == 0 && tm0 + Cfg::BM <= M && tn0 + Cfg::BN <= N;
        v = vn;
    }
}

}  // namespace lpgemm
