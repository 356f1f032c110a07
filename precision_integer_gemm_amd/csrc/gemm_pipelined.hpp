// gemm_pipelined.hpp -- block-tiled int8-MFMA GEMM for gfx950 with a
// multi-stage direct-to-LDS pipeline (both operand formats).
//
// C[M,N] = A[M,K] . B[N,K]^T ("NT": operand rows contiguous in K, as in the
// int4 example's T.gemm(..., transpose_B=True) and the w4a8 example).
//
// Staging (a1).  Operand tiles go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: every lane moves 16 bytes, a wave instruction
// fills 1 KB of LDS at M0 + 16 * lane.  Each lane picks the global 16-byte
// chunk that lands, in LDS, at its row-major position with the 16-byte
// columns XOR-swizzled, so fragment reads are free of bank conflicts.  The
// buffer resource's range check returns zeros for rows past the matrix end,
// and lanes whose chunk lies past K use an out-of-range offset, so tails are
// zero-filled without branches.  All STAGES slots of an LDS ring are kept in
// flight; one barrier per K tile, placed before the tile's last 64-k step so
// the next tile's first fragment reads overlap that step's MFMAs, and the
// copy that refills the freed slot goes out after those MFMAs.  Raw
// fragments are double-buffered in registers one step ahead.  The loads are
// invisible to the compiler, so the kernel issues its own vmcnt waits.
//
// Contraction (a2, a3).  Each wave owns FN x FM blocks of 32x32 outputs.  Per
// 64 k it reads one 16-byte LDS vector per 4-bit operand block (32 nibbles ->
// two MFMA operands, unpacked x16 in registers) or two per int8 block, and
// issues v_mfma_i32_32x32x32_i8 twice per block.  B is the MFMA's row operand
// and A its column operand, so the accumulators hold C^T and each lane ends
// with four consecutive n of one m (16-byte stores).
//
// Epilogue (a5): exact >> 8 (int4 x int4) or >> 4 (W4A8), masked stores of
// int32, or of the per-row / per-column scaled fp32, bf16 or fp16 value.
//
// Tile order: persistent workgroups loop over tiles; the next tile's first
// loads are issued before the current tile's stores, so the stores drain
// under the next tile's work.  Workgroup b runs on XCD b % 8 and tiles are
// renumbered so each XCD walks a compact band of C (shared A rows and B
// columns in its L2).
//
// Split K (SPLIT, int32 output, one tile per workgroup): the grid is the tiles
// times `chunks` K ranges of kc; workgroup b contracts range b / tiles of tile
// b % tiles and stores its sums into slice b / tiles of an M x N int32
// workspace (epi.out), which a second kernel sums into C.
//
// Per-K-block scales (SBP > 0, integer formats, the tutorial's
// gemm_blockscaled read for integer operands): the int32 accumulators hold
// one block's partial sum; where a block of g k ends, each element becomes
// ((float)C_j * SFA[m][j]) * SFB[n][j] and is added to an fp32 accumulator
// (started at -0, so the first block's term is taken as it is), and the
// int32 accumulators restart.  The stage copy also brings the stage's blocks'
// scale rows into LDS (4-byte DMA, one float per lane), in a ring of
// STAGES + 1 slots so that a wave still flushing a tile's last block never
// races the refill of that block's slot.  SBP is the number of blocks per
// 128-k stage: 4 (g = 32), 2 (g = 64) or 1 (g >= 128, the stage inside one
// block).  With g = 32 each MFMA must contract one whole block, so the
// fragments are read with a different lane-to-k map: lanes 0-31 feed k 0-15
// and lanes 32-63 k 16-31 of the first instruction (k 32-63: the second),
// two 8-byte LDS reads per packed row instead of one 16-byte read.
//
// Requirements (checked on the host): K % 32 == 0, 16-byte aligned bases,
// M, N < 2^31, K <= 131070; with SPLIT kc % 256 == 0 and a grid of exactly
// tiles x ranges; with SBP g = 128 / SBP (SBP > 1) or g >= 128 (SBP = 1), a
// power of two.
#pragma once

#include "device_common.hpp"

namespace lpgemm {

template <int VAR, int FM, int FN, int WM, int WN, int BK, int STAGES, int SBP = 0>
struct PipeCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = WM * FM * 32;
    static constexpr int BN = WN * FN * 32;
    static constexpr int RA = (VAR == I4I4) ? BK / 2 : BK;  // LDS bytes per A row
    static constexpr int RB = is_fp8(VAR) ? BK : BK / 2;   // LDS bytes per B row
    static constexpr int CPR_A = RA / 16;
    static constexpr int CPR_B = RB / 16;
    static constexpr int A_BYTES = BM * RA;
    static constexpr int B_BYTES = BN * RB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Without block scales: two slots for a tile's per-row / per-column
    // scale vectors (scaled outputs), BM + BN floats rounded up to whole
    // 64-float DMA instructions.
    static constexpr int CHAN_SLOT = 4 * ((BM + BN + 63) / 64 * 64);
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + (SBP == 0 ? 2 * CHAN_SLOT : 0);
    static constexpr int NA = A_BYTES / 1024 / kWaves;  // DMA instructions per wave per stage
    static constexpr int NB = B_BYTES / 1024 / kWaves;
    static constexpr int SHIFT = (VAR == I4I4) ? 8 : 4;
    // Block-scale ring: SBP blocks' SFA rows (BM floats each) and SFB rows
    // (BN floats each) per slot, padded to whole 4-byte DMA instructions
    // (NS per wave per stage), STAGES + 1 slots.
    static constexpr int SCALES = (BM + BN) * SBP;
    static constexpr int NS = SBP ? (SCALES + 64 * kWaves - 1) / (64 * kWaves) : 0;
    static constexpr int SCALE_SLOT_BYTES = NS * 64 * kWaves * 4;
    static constexpr int SCALE_SLOTS = SBP ? STAGES + 1 : 0;
    static constexpr int LDS_BYTES_ALL = LDS_BYTES + SCALE_SLOTS * SCALE_SLOT_BYTES;
    static_assert(SBP == 0 || SBP == 1 || SBP == 2 || SBP == 4, "blocks per stage");
    static_assert(SBP == 0 || (BK == 128 && !is_fp8(VAR)), "block scales: integer formats, 128-k stages");
    static_assert(SBP == 0 || (BM * SBP) % 64 == 0, "a scale DMA instruction must not straddle SFA and SFB");
    static_assert(BK % 64 == 0, "BK must be a multiple of 64");
    static_assert(NA * 1024 * kWaves == A_BYTES && NB * 1024 * kWaves == B_BYTES,
                  "each wave must issue whole 1 KB DMA instructions");
    static_assert(CPR_A <= 16 && CPR_B <= 16, "row too long for the swizzle");
    static constexpr bool kFits = STAGES >= 2 && LDS_BYTES_ALL <= 160 * 1024;
};

// Position of 16-byte chunk `col` of tile row `row` in a row-major LDS tile
// of CPR chunks per row.  The XOR spreads the 16 rows that one 256-byte LDS
// line serves across distinct bank groups.
template <int CPR>
__device__ __forceinline__ int lds_chunk(int row, int col)
{
    constexpr int rows_per_256 = 16 / CPR;
    return row * CPR + (col ^ ((row / rows_per_256) % CPR));
}

template <int VAR, int FM, int FN, int WM, int WN, int BK, int STAGES, int OUT, bool SPLIT = false,
          int SBP = 0>
__global__ __launch_bounds__(64 * WM * WN, (FM * FN <= 8 && (SBP == 0 || WM * WN == 4)) ? 2 : 1) void gemm_pipelined_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, Epilogue epi, int M, int N,
    int K, int tiles_m, int tiles_n, int xcds, int kc)
{
    static_assert(!SPLIT || OUT == OUT_I32, "split K adds int32 partial sums");
    static_assert(SBP == 0 || (!SPLIT && (OUT == OUT_F32 || OUT == OUT_BF16 || OUT == OUT_F16)),
                  "block scales: whole K per tile, float output");
    using Cfg = PipeCfg<VAR, FM, FN, WM, WN, BK, STAGES, SBP>;
    constexpr bool K32 = SBP == 4;  // g = 32: one block per MFMA instruction
    static_assert(Cfg::kFits, "LDS ring does not fit in 160 KB");
    constexpr int RA = Cfg::RA, RB = Cfg::RB, CPR_A = Cfg::CPR_A, CPR_B = Cfg::CPR_B;
    constexpr int NA = Cfg::NA, NB = Cfg::NB;
    constexpr int STEPS = BK / 64;
    constexpr int NS = Cfg::NS;
    constexpr int kPerStage = NA + NB + NS;  // DMA instructions per wave per stage
    constexpr int kPrologue = STAGES;  // stages loaded before a tile's first step
    // 16-byte stores per wave for a tile with no edge (a lower bound on the
    // vector-memory instructions its epilogue issues).
    constexpr int kStores = FN * FM * 4;
    extern __shared__ __align__(1024) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;

    const uint32_t lda = (VAR == I4I4) ? (uint32_t)K / 2 : (uint32_t)K;  // global row bytes
    const uint32_t ldb = is_fp8(VAR) ? (uint32_t)K : (uint32_t)K / 2;
    // This workgroup's K range [k0, k0 + klen) (all of K unless SPLIT), and its
    // offset and length in bytes of an A row and a B row.
    const int nblocks = tiles_m * tiles_n;
    const int chunk = SPLIT ? (int)blockIdx.x / nblocks : 0;
    const int k0 = chunk * kc;
    const int klen = SPLIT ? min(kc, K - k0) : K;
    const uint32_t a_k0 = (VAR == I4I4) ? (uint32_t)k0 / 2 : (uint32_t)k0;
    const uint32_t b_k0 = is_fp8(VAR) ? (uint32_t)k0 : (uint32_t)k0 / 2;
    const uint32_t a_len = (VAR == I4I4) ? (uint32_t)klen / 2 : (uint32_t)klen;
    const uint32_t b_len = is_fp8(VAR) ? (uint32_t)klen : (uint32_t)klen / 2;
    const int ktiles = (klen + BK - 1) / BK;
    // Where the tile's results go: C, or this range's workspace slice.
    Epilogue epo = epi;
    if (SPLIT) epo.out = static_cast<int32_t *>(epi.out) + (int64_t)chunk * M * N;

    // Per-lane source of each DMA instruction: tile row and 16-byte column.
    uint32_t a_off[NA], a_col[NA], b_off[NB], b_col[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int q = (wave * NA + i) * 64 + lane;
        const int row = q / CPR_A, slot = q % CPR_A;
        const int col = slot ^ ((row / (16 / CPR_A)) % CPR_A);
        a_col[i] = 16u * col;
        a_off[i] = row * lda + a_col[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int q = (wave * NB + i) * 64 + lane;
        const int row = q / CPR_B, slot = q % CPR_B;
        const int col = slot ^ ((row / (16 / CPR_B)) % CPR_B);
        b_col[i] = 16u * col;
        b_off[i] = row * ldb + b_col[i];
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    // Block scales: DMA instruction i of this wave moves scale elements e =
    // (wave * NS + i) * 64 + lane of the slot: SFA[m0 + r][j] for e < BM * SBP
    // (r = e % BM, block jj = e / BM of the stage), then SFB[n0 + r][j].
    // s_off is the byte offset of the element's row inside its table tile;
    // the stage adds 4 j.  Elements past the slot's SCALES are padding.
    const int nb = SBP ? epi.nb : 0, lg = SBP ? epi.lg : 0;
    uint32_t s_off[NS > 0 ? NS : 1];
    int s_jj[NS > 0 ? NS : 1];
    bool s_live[NS > 0 ? NS : 1], s_isb[NS > 0 ? NS : 1];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int e0 = (wave * NS + i) * 64;  // wave-uniform
        const int e = e0 + lane;
        s_isb[i] = e0 >= Cfg::BM * SBP;
        s_live[i] = e < Cfg::SCALES;
        const int eb = s_isb[i] ? e - Cfg::BM * SBP : e;
        const int rows = s_isb[i] ? Cfg::BN : Cfg::BM;
        s_jj[i] = eb / rows;
        s_off[i] = (uint32_t)(eb % rows) * (uint32_t)nb * 4u;
    }

    // Persistent tile loop: workgroup b takes tiles b, b + G, b + 2G, ... (G =
    // number of workgroups).  Tiles are renumbered so that each XCD
    // (workgroup b runs on XCD b % xcds) walks a contiguous range of tile
    // ids, taken in bands of 4 tile rows, which keeps the A rows and B columns
    // its workgroups share in that XCD's L2.
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

    int v = (int)blockIdx.x - chunk * nblocks;
    int m0, n0;
    tile_origin(v, m0, n0);
    // Per-row / per-column scales of a scaled integer output (one K block).
    constexpr bool kChan = OUT != OUT_I32 && SBP == 0 && !is_fp8(VAR);
    i32x4 rsrc_a, rsrc_b, rsrc_sa, rsrc_sb;
    auto set_rsrc = [&]() {
        rsrc_a = make_rsrc(A + (int64_t)m0 * lda, (uint32_t)min(Cfg::BM, M - m0) * lda);
        rsrc_b = make_rsrc(B + (int64_t)n0 * ldb, (uint32_t)min(Cfg::BN, N - n0) * ldb);
        if constexpr (SBP > 0) {
            rsrc_sa = make_rsrc(epi.scale_a + (int64_t)m0 * nb, (uint32_t)min(Cfg::BM, M - m0) * nb * 4u);
            rsrc_sb = make_rsrc(epi.scale_b + (int64_t)n0 * nb, (uint32_t)min(Cfg::BN, N - n0) * nb * 4u);
        } else if constexpr (kChan) {
            rsrc_sa = make_rsrc(epi.scale_a + m0, (uint32_t)min(Cfg::BM, M - m0) * 4u);
            rsrc_sb = make_rsrc(epi.scale_b + n0, (uint32_t)min(Cfg::BN, N - n0) * 4u);
        }
    };
    set_rsrc();

    // DMA of stage kt (A's rows, then B's) into its ring slot.  Past K every
    // offset is out of range: the slot fills with zeros.
    auto issue_stage = [&](int kt) {
        const uint32_t base = lds0 + (uint32_t)(kt % STAGES) * Cfg::STAGE_BYTES;
        const uint32_t ka = (uint32_t)kt * RA, kb = (uint32_t)kt * RB;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const uint32_t off = (ka + a_col[i] < a_len) ? a_off[i] + a_k0 + ka : kOutOfRange;
            dma16(rsrc_a, off, base + (uint32_t)(wave * NA + i) * 1024u);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint32_t off = (kb + b_col[i] < b_len) ? b_off[i] + b_k0 + kb : kOutOfRange;
            dma16(rsrc_b, off, base + Cfg::A_BYTES + (uint32_t)(wave * NB + i) * 1024u);
        }
        if constexpr (SBP > 0) {
            // the stage's blocks: jb (the block of its first k) .. jb + SBP - 1
            const uint32_t sbase = lds0 + (uint32_t)(STAGES * Cfg::STAGE_BYTES) +
                                   (uint32_t)(kt % (STAGES + 1)) * Cfg::SCALE_SLOT_BYTES;
            const int jb = (kt * BK) >> lg;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int j = jb + s_jj[i];
                const uint32_t off = (s_live[i] && j < nb) ? s_off[i] + 4u * (uint32_t)j : kOutOfRange;
                dma4(s_isb[i] ? rsrc_sb : rsrc_sa, off, sbase + (uint32_t)(wave * NS + i) * 256u);
            }
        }
    };

    const int h = lane >> 5;    // which 16-k half of an MFMA operand this lane feeds
    const int r32 = lane & 31;  // operand row inside a 32-row block

    // Raw (still packed / int8 / fp8) fragments of one 64-k step, as read
    // from LDS: 16 bytes of a 4-bit row, 32 bytes of a byte-wide row.
    constexpr int AV = (VAR == I4I4) ? 1 : 2;  // 16-byte vectors per A block row
    constexpr int BV = is_fp8(VAR) ? 2 : 1;   // 16-byte vectors per B block row
    struct Frags {
        i32x4 b[FN][BV];
        i32x4 a[FM][AV];
    };
    // g = 32: per packed row the two 8-byte halves 8h of the step's two
    // 16-byte chunks (k 16h..16h+15 and 32+16h..32+16h+15 of the step), per
    // int8 row chunks h and 2 + h.
    auto read_frags = [&](int slot, int step, Frags &f) {
        const uint8_t *sa = smem + slot * Cfg::STAGE_BYTES;
        const uint8_t *sb = sa + Cfg::A_BYTES;
        if constexpr (K32) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = (wn * FN + fn) * 32 + r32;
                const u32x2 x = *reinterpret_cast<const u32x2 *>(sb + 16 * lds_chunk<CPR_B>(row, 2 * step) + 8 * h);
                const u32x2 y =
                    *reinterpret_cast<const u32x2 *>(sb + 16 * lds_chunk<CPR_B>(row, 2 * step + 1) + 8 * h);
                f.b[fn][0] = i32x4{(int32_t)x.x, (int32_t)x.y, (int32_t)y.x, (int32_t)y.y};
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = (wm * FM + fm) * 32 + r32;
                if constexpr (VAR == I4I4) {
                    const u32x2 x =
                        *reinterpret_cast<const u32x2 *>(sa + 16 * lds_chunk<CPR_A>(row, 2 * step) + 8 * h);
                    const u32x2 y =
                        *reinterpret_cast<const u32x2 *>(sa + 16 * lds_chunk<CPR_A>(row, 2 * step + 1) + 8 * h);
                    f.a[fm][0] = i32x4{(int32_t)x.x, (int32_t)x.y, (int32_t)y.x, (int32_t)y.y};
                } else {
#pragma unroll
                    for (int v = 0; v < AV; ++v)
                        f.a[fm][v] = *reinterpret_cast<const i32x4 *>(
                            sa + 16 * lds_chunk<CPR_A>(row, 4 * step + 2 * v + h));
                }
            }
            return;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int row = (wn * FN + fn) * 32 + r32;
#pragma unroll
            for (int v = 0; v < BV; ++v) {
                const int col = is_fp8(VAR) ? 4 * step + 2 * h + v : 2 * step + h;
                f.b[fn][v] = *reinterpret_cast<const i32x4 *>(sb + 16 * lds_chunk<CPR_B>(row, col));
            }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = (wm * FM + fm) * 32 + r32;
#pragma unroll
            for (int v = 0; v < AV; ++v) {
                const int col = (VAR == I4I4) ? 2 * step + h : 4 * step + 2 * h + v;
                f.a[fm][v] = *reinterpret_cast<const i32x4 *>(sa + 16 * lds_chunk<CPR_A>(row, col));
            }
        }
    };

    // Integer accumulators for the int4 / int8 formats, fp32 for fp8.
    using Acc = typename std::conditional<is_fp8(VAR), f32x16, i32x16>::type;
    Acc acc[FN][FM];
    // Block scales: fp32 accumulators, and the scale rows of one block.
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x16 facc[SBP > 0 ? FN : 1][SBP > 0 ? FM : 1];
    // fa += ((float)C_j * SFA) * SFB element by element, each operation a
    // binary32 one rounding to nearest even; c holds C_j << SHIFT exactly.
    // PRE: sa already holds SFA * 2^-SHIFT, and (float)c * sa is then the
    // same real number as C_j * SFA, so it rounds to the same binary32 value
    // with one operation less (see prescale).
    auto add_block = [&](auto pre, f32x16 &fa, const i32x16 &c, float sa,
                         const f32x4 (&sb)[4]) __attribute__((always_inline)) {
        constexpr bool PRE = decltype(pre)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float t = PRE ? (float)c[r] : (float)(c[r] >> Cfg::SHIFT);
            const float y = t * sa;
            float z = y * sb[r / 4][r % 4];
            asm volatile("" : "+v"(z));  // two separate roundings, no fused operation
            fa[r] = fa[r] + z;
        }
    };
    // Fold 2^-SHIFT into this wave's SFA values when that is exact for every
    // lane: (float)c is exact while |c| <= 2^24, which |C_j| <= 64 g (int4 x
    // int4) or 1024 g (W4A8) guarantees for g <= 1024, and SFA * 2^-SHIFT is
    // exact unless it falls below the normal range.  Wave-uniform answer.
    auto prescale = [&](float (&sa)[FM]) __attribute__((always_inline)) {
        bool ok = lg <= 10;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const float a = __builtin_fabsf(sa[fm]);
            ok = ok && (a == 0.f || !(a < 0x1p-126f * (float)(1 << Cfg::SHIFT)));
        }
        if (!__all(ok)) return false;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) sa[fm] *= 1.0f / (float)(1 << Cfg::SHIFT);
        return true;
    };
    using Pre = std::true_type;
    using Raw = std::false_type;
    // Add block j (a block of the stage of K tile kt) held in acc to facc and
    // clear acc: SFA[m][j] of this lane's rows, SFB[n][j] of its columns (four
    // groups of four), read from the stage's scale slot.
    auto flush = [&](int kt, int j) __attribute__((always_inline)) {
        if constexpr (SBP > 0) {
            const int jj = j - ((kt * BK) >> lg);
            const float *slot = reinterpret_cast<const float *>(smem + STAGES * Cfg::STAGE_BYTES +
                                                                (kt % (STAGES + 1)) * Cfg::SCALE_SLOT_BYTES);
            const float *ta = slot + jj * Cfg::BM;
            const float *tb = slot + Cfg::BM * SBP + jj * Cfg::BN;
            float sa[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sa[fm] = ta[(wm * FM + fm) * 32 + r32];
            auto body = [&](auto pre) __attribute__((always_inline)) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    f32x4 sb[4];
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
                        sb[rg] = *reinterpret_cast<const f32x4 *>(tb + (wn * FN + fn) * 32 + 8 * rg + 4 * h);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
                        add_block(pre, facc[fn][fm], acc[fn][fm], sa[fm], sb);
                        acc[fn][fm] = Acc{};
                    }
                }
            };
            if (prescale(sa))
                body(Pre{});
            else
                body(Raw{});
        }
    };

    // Unpack and contract one 64-k step: per block two 32x32x32 int8 MFMAs,
    // or one 32x32x64 fp8 MFMA (lane l: 32 consecutive k, 32 (l / 32) onward).
    auto compute = [&](const Frags &f, int kt, int st) {
        (void)kt;
        (void)st;
        if constexpr (is_fp8(VAR)) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = mfma_32x32x64_fp8<VAR == BF8 ? 1 : 0>(f.b[fn][0], f.b[fn][BV - 1], f.a[fm][0],
                                                    f.a[fm][AV - 1], acc[fn][fm]);
        } else {
            i32x4 a_lo[FM], a_hi[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                i32x4 b_lo, b_hi;
                unpack_chunk<VAR == W4A8>(f.b[fn][0], b_lo, b_hi);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if (fn == 0) {
                        if (VAR == I4I4) {
                            unpack_chunk<false>(f.a[fm][0], a_lo[fm], a_hi[fm]);
                        } else {
                            a_lo[fm] = f.a[fm][0];
                            a_hi[fm] = f.a[fm][AV - 1];
                        }
                    }
                    acc[fn][fm] = mfma_32x32x32(b_lo, a_lo[fm], acc[fn][fm]);
                    acc[fn][fm] = mfma_32x32x32(b_hi, a_hi[fm], acc[fn][fm]);
                }
            }
        }
    };

    // One 64-k step with block scales.  g = 32: each instruction contracts
    // one whole block (blocks j1 and j1 + 1) from zero and is added at once;
    // g >= 64: the step's products go into the int32 accumulators, which are
    // added and cleared where the step ends block j (or ends K).  Blocks at
    // or past nb (the zero-filled steps after K) are skipped.
    auto compute_scaled = [&](const Frags &f, int kt, int st) __attribute__((always_inline)) {
        if constexpr (SBP > 0) {
            const int ks = kt * BK + 64 * st;  // the step's first k
            if constexpr (K32) {
                const int j1 = ks >> 5;
                if (j1 >= nb) return;
                i32x4 a_lo[FM], a_hi[FM], b_lo[FN], b_hi[FN];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if (VAR == I4I4) {
                        unpack_chunk<false>(f.a[fm][0], a_lo[fm], a_hi[fm]);
                    } else {
                        a_lo[fm] = f.a[fm][0];
                        a_hi[fm] = f.a[fm][AV - 1];
                    }
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    unpack_chunk<VAR == W4A8>(f.b[fn][0], b_lo[fn], b_hi[fn]);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_32x32x32(b_lo[fn], a_lo[fm], i32x16{});
                }
                flush(kt, j1);
                if (j1 + 1 < nb) {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_32x32x32(b_hi[fn], a_hi[fm], i32x16{});
                    flush(kt, j1 + 1);
                }
            } else {
                compute(f, kt, st);
                const int j = ks >> lg;
                const bool ends = ((ks + 64) & ((1 << lg) - 1)) == 0 || ks + 64 >= K;
                if (j < nb && ends) {
                    // all scale rows first, then the unfolded terms: with two
                    // waves of 64 x 64 per SIMD this measured faster than the
                    // folded form and per-column-group reads (4096^3 W4A8, g =
                    // 128: 159 against 176 us)
                    const int jj = j - ((kt * BK) >> lg);
                    const float *slot = reinterpret_cast<const float *>(
                        smem + STAGES * Cfg::STAGE_BYTES + (kt % (STAGES + 1)) * Cfg::SCALE_SLOT_BYTES);
                    const float *ta = slot + jj * Cfg::BM;
                    const float *tb = slot + Cfg::BM * SBP + jj * Cfg::BN;
                    float sa[FM];
                    f32x4 sb[FN][4];
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) sa[fm] = ta[(wm * FM + fm) * 32 + r32];
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg)
                            sb[fn][rg] =
                                *reinterpret_cast<const f32x4 *>(tb + (wn * FN + fn) * 32 + 8 * rg + 4 * h);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int fm = 0; fm < FM; ++fm) {
                            add_block(Raw{}, facc[fn][fm], acc[fn][fm], sa[fm], sb[fn]);
                            acc[fn][fm] = Acc{};
                        }
                }
            }
        }
    };
    auto step = [&](const Frags &f, int kt, int st) {
        if constexpr (SBP > 0)
            compute_scaled(f, kt, st);
        else
            compute(f, kt, st);
    };

    // W4A8 with int32 output on 256-tiles: B is unpacked one step ahead, into
    // buffer (step % 2), so the next step's unpack runs beside this step's
    // MFMAs (measured 1.6-2.9% faster; the scaled instances, nearer the
    // register limit, unpack within the step).
    constexpr bool kPreB = VAR == W4A8 && SBP == 0 && OUT == OUT_I32 && !SPLIT && FM * FN == 8;
    static_assert(!kPreB || STEPS % 2 == 0, "the unpack buffers alternate within a K tile");
    i32x4 ubl[kPreB ? 2 : 1][FN], ubh[kPreB ? 2 : 1][FN];
    auto unpack_b = [&](const Frags &f, int buf) __attribute__((always_inline)) {
        if constexpr (kPreB) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) unpack_chunk<true>(f.b[fn][0], ubl[buf][fn], ubh[buf][fn]);
        }
    };
    auto compute_pre = [&](const Frags &f, int buf) __attribute__((always_inline)) {
        if constexpr (kPreB) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    acc[fn][fm] = mfma_32x32x32(ubl[buf][fn], f.a[fm][0], acc[fn][fm]);
                    acc[fn][fm] = mfma_32x32x32(ubh[buf][fn], f.a[fm][AV - 1], acc[fn][fm]);
                }
        }
    };

    // Wait until this wave's loads of the stage issued `after` stages before
    // the newest one have landed (loads complete in issue order).
    auto wait_tiles_after = [&](int after) {
        if (after >= 4)
            wait_vmcnt<4 * kPerStage>();
        else if (after >= 3)
            wait_vmcnt<3 * kPerStage>();
        else if (after == 2)
            wait_vmcnt<2 * kPerStage>();
        else if (after == 1)
            wait_vmcnt<kPerStage>();
        else
            wait_vmcnt<0>();
    };

    // Stages 0 .. kPrologue-1 of the first tile.  Slots past the last K tile
    // are filled too (with zeros: every offset is out of range), which keeps
    // the number of loads in flight the same in every iteration.
    // Scaled outputs: a tile's scale vectors go into LDS slot p with the
    // tile's first copies, element e = 64 wave + lane being scale_a[m0 + e]
    // for e < BM, then scale_b[n0 + e - BM] (zeros past M and N).  The
    // epilogue reads them from LDS, so no global load of its own has to be
    // waited for behind the next tile's copies.
    const uint32_t lds_chan = lds0 + (uint32_t)(STAGES * Cfg::STAGE_BYTES);
    int par = 0;  // slot of the current tile's scales
    auto issue_scales = [&](int p) {
        if constexpr (kChan) {
            static_assert(Cfg::BM % 64 == 0, "a scale DMA instruction must not straddle the two vectors");
            for (int e0 = wave * 64; e0 < Cfg::BM + Cfg::BN; e0 += 64 * Cfg::kWaves) {  // wave-uniform
                const bool isb = e0 >= Cfg::BM;
                const uint32_t off = (uint32_t)((isb ? e0 - Cfg::BM : e0) + lane) * 4u;
                dma4(isb ? rsrc_sb : rsrc_sa, off, lds_chan + (uint32_t)(p * Cfg::CHAN_SLOT + e0 * 4));
            }
        }
    };
    issue_scales(0);
#pragma unroll
    for (int s = 0; s < kPrologue; ++s) issue_stage(s);
    bool stores_pending = false;  // a full tile's stores were issued after the prologue

    for (;;) {
        // Stage 0 of this tile has landed.  The previous tile's stores were
        // issued after this tile's prologue loads, so they may stay in flight.
        if (stores_pending)
            wait_vmcnt<(kPrologue - 1) * kPerStage + kStores>();
        else
            wait_vmcnt<(kPrologue - 1) * kPerStage>();
        lds_barrier();

#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = Acc{};
        if constexpr (SBP > 0) {
            // -0 + x == x for every x: the first block's term is taken as it is
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) facc[i][j][r] = -0.0f;
        }
        Frags cur, nxt;
        read_frags(0, 0, cur);
        unpack_b(cur, 0);

        // Steady state: every K tile but the last.  The tile's last step waits
        // for tile kt+1, passes the barrier (every wave is done reading tile
        // kt), reads step 0 of tile kt+1, issues its MFMAs and then refills
        // tile kt's slot with tile kt+STAGES.
        for (int kt = 0; kt + 1 < ktiles; ++kt) {
            const int slot = kt % STAGES;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                if (st + 1 < STEPS) {
                    read_frags(slot, st + 1, nxt);
                } else {
                    wait_tiles_after(STAGES - 2);
                    lds_barrier();
                    read_frags((kt + 1) % STAGES, 0, nxt);
                }
                if constexpr (kPreB) {
                    compute_pre(cur, st & 1);
                    unpack_b(nxt, (st + 1) & 1);
                } else {
                    step(cur, kt, st);
                }
                if (st + 1 == STEPS) issue_stage(kt + STAGES);
                cur = nxt;
            }
        }
        // Last K tile.
        {
            const int slot = (ktiles - 1) % STAGES;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                if (st + 1 < STEPS) read_frags(slot, st + 1, nxt);
                if constexpr (kPreB) {
                    compute_pre(cur, st & 1);
                    if (st + 1 < STEPS) unpack_b(nxt, (st + 1) & 1);
                } else {
                    step(cur, ktiles - 1, st);
                }
                cur = nxt;
            }
        }
        wait_vmcnt<0>();  // the zero-fill loads past the end

        const int tm0 = m0, tn0 = n0;
        const int tpar = par;
        const int vn = v + (int)gridDim.x;
        // Epilogue: lane holds C[m][n .. n+3] for m = l%32 of each column block.
        auto store_tile = [&]() {
            if constexpr (SBP > 0) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
                        const int m = tm0 + (wm * FM + fm) * 32 + r32;
                        if (m >= M) continue;
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) {
                            const int n = tn0 + (wn * FN + fn) * 32 + 8 * rg + 4 * h;
                            const float c[4] = {facc[fn][fm][4 * rg + 0], facc[fn][fm][4 * rg + 1],
                                                facc[fn][fm][4 * rg + 2], facc[fn][fm][4 * rg + 3]};
                            store_row4f<OUT>(epi, m, N, n, c);
                        }
                    }
                return;
            }
            // Scales from this tile's LDS slot (one per row block, four per
            // column group).
            float sa[FM], sb[FN][4][4];
            if constexpr (kChan) {
                const float *ss =
                    reinterpret_cast<const float *>(smem + STAGES * Cfg::STAGE_BYTES + tpar * Cfg::CHAN_SLOT);
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
                        if constexpr (is_fp8(VAR)) {
                            const float c[4] = {acc[fn][fm][4 * rg + 0], acc[fn][fm][4 * rg + 1],
                                                acc[fn][fm][4 * rg + 2], acc[fn][fm][4 * rg + 3]};
                            store_row4f<OUT>(epi, m, N, n, c);
                        } else {
                            const i32x4 c = i32x4{acc[fn][fm][4 * rg + 0], acc[fn][fm][4 * rg + 1],
                                                  acc[fn][fm][4 * rg + 2], acc[fn][fm][4 * rg + 3]} >>
                                            Cfg::SHIFT;
                            store_row4<OUT>(epo, m, N, n, c, sa[fm], sb[fn][rg]);
                        }
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
        // (shifted integers, or binary32 bits for fp8 operands; padded rows),
        // then every wave stores rows of it.
        constexpr bool kStageC = Cfg::BN == 256 && SBP == 0;
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
                reinterpret_cast<const float *>(smem + STAGES * Cfg::STAGE_BYTES + tpar * Cfg::CHAN_SLOT);
            float sb4[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kChan) {
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
                            i32x4 c;
                            if constexpr (is_fp8(VAR)) {  // binary32 results, staged as their bits
#pragma unroll
                                for (int i = 0; i < 4; ++i) c[i] = __float_as_int(acc[fn][fm][4 * rg + i]);
                            } else {
                                c = i32x4{acc[fn][fm][4 * rg + 0], acc[fn][fm][4 * rg + 1],
                                          acc[fn][fm][4 * rg + 2], acc[fn][fm][4 * rg + 3]} >>
                                    Cfg::SHIFT;
                            }
                            *reinterpret_cast<i32x4 *>(smem + (rb - p0 + sr32) * kPitch + 4 * col) = c;
                        }
                }
                lds_barrier();
                for (int r = p0 + wave; r < p0 + kRows && r < Cfg::BM; r += Cfg::kWaves) {
                    const int m = tm0 + r;
                    if (m >= M) break;
                    const i32x4 c = *reinterpret_cast<const i32x4 *>(smem + (r - p0) * kPitch + 16 * sl);
                    if constexpr (is_fp8(VAR)) {
                        const float cf[4] = {__int_as_float(c[0]), __int_as_float(c[1]), __int_as_float(c[2]),
                                             __int_as_float(c[3])};
                        store_row4f<OUT>(epo, m, N, tn0 + 4 * sl, cf);
                    } else {
                        store_row4<OUT>(epo, m, N, tn0 + 4 * sl, c, kChan ? ss[r] : 0.f, sb4);
                    }
                }
            }
          }
        };
        // The next tile's loads go out before this tile's stores (one store
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
