// gemm_skinny.hpp -- narrow-M kernel for gfx950 (decode-like shapes), for
// W4A8 and for int4 x int4.
//
// For M <= 16 the product is bound by reading the packed weights B once from
// HBM, so the kernel is built around streaming B at full bandwidth.  A (int8,
// or packed int4 unpacked x16 when it is loaded) stays in registers.
#pragma once

#include "device_common.hpp"

namespace lpgemm {

// B reaches LDS through direct-to-LDS buffer loads in which every instruction
// reads 1 KB of one row, so HBM sees long row-linear bursts (a lane-per-row
// register load, 16 rows x 64 bytes per instruction, streams markedly slower).
// The loads carry the non-temporal hint: each byte of B is read once.
//
//   * workgroup = KW waves, one per compute unit, walking strips of 16 rows
//     of B (grid-stride); two LDS strip buffers, the next strip's loads in
//     flight while the current strip is contracted;
//   * strip layout in LDS: row-major, 16-byte chunks, chunk c of row r stored
//     at position c ^ (r % 16) when a row holds a multiple of 16 chunks (the
//     MFMA fragment reads of 16 rows at one k then hit 16 distinct bank
//     groups); each DMA instruction still covers one contiguous 1 KB span;
//   * wave w owns the w-th slice of K (KSTEPS steps of 128 logical k) for the
//     whole kernel and keeps the matching A fragments (rows zero-padded to
//     16, read once) in registers; fragments of B come from LDS with
//     ds_read_b128, are unpacked in registers and contracted with
//     v_mfma_i32_16x16x64_i8, B as the MFMA's 16-row operand and A as its
//     16-column operand (the w4a8 page's kernel also puts the dequantised B
//     first and produces C^T), so each lane ends with four consecutive n of
//     one m;
//   * the KW partial tiles of a strip are summed in LDS in a fixed order by
//     one wave (rotating) after the next iteration's barrier, so one barrier
//     per strip suffices and C stores overlap the next strip's work.
//
// Row groups: M up to 64 is taken as ceil(M / 16) groups of 16 rows of A, each
// by its own equal group of workgroups over all strips; workgroups b and
// b + (a multiple of 8) run on one XCD, so the groups' reads of a strip after
// the first are served by that XCD's L2 or the MALL.  Each group writes its
// own rows of C.
//
// Split K (SPLIT, int32 output only): K longer than one workgroup's waves
// cover is cut into ranges of kc; every row group's workgroups are split again
// into `chunks` equal sets, set c contracting k in [c kc, (c + 1) kc) for its
// share of the strips (its A range loaded once), and every strip's sum is
// added into C, zeroed beforehand, with int32 atomic adds -- exact and
// independent of order.
//
// Requirements (checked on the host): M <= 64, K % 32 == 0, 16-byte aligned
// bases, N * K / 2 < 2^31, KW * KSTEPS * 128 >= kc, kc % 32 == 0, at most 256
// workgroups, a multiple of (row groups x K ranges) with a multiple of 8
// workgroups per set.
template <int KW, int KSTEPS>
struct SkinnyCfg {
    static constexpr int kBufBytes = KW * KSTEPS * 1024;  // one strip (16 rows x K/2 bytes, padded)
    static constexpr int kRedBytes = 2 * KW * 64 * 16;
    static constexpr int kLdsBytes = 2 * kBufBytes + kRedBytes;
    static_assert(kLdsBytes <= 160 * 1024, "strip buffers exceed the LDS");
};

template <int VAR, int KW, int KSTEPS, int OUT, bool SPLIT, bool WHOLE_A = false>
__global__ __launch_bounds__(64 * KW) void gemm_skinny_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, Epilogue epi, int M, int N, int K,
    int kc)
{
    static_assert(!SPLIT || OUT == OUT_I32, "split K adds int32 partial sums");
    static_assert(VAR == W4A8 || VAR == I4I4, "4-bit B with an int8 or int4 A");
    static_assert(!WHOLE_A || VAR == W4A8, "whole-line A loads: int8 A");
    // x16 pre-scale of each 4-bit operand, removed exactly at the end
    constexpr int kShift = VAR == I4I4 ? 8 : 4;
    using Cfg = SkinnyCfg<KW, KSTEPS>;
    extern __shared__ __align__(1024) uint8_t smem[];
    i32x4 *red = reinterpret_cast<i32x4 *>(smem + 2 * Cfg::kBufBytes);  // [2][KW][64]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int strips = (N + 15) / 16;
    // This workgroup's K range [k0, k0 + klen) and its share of the strips.
    const int chunks = SPLIT ? (K + kc - 1) / kc : 1;
    const int mgroups = (M + 15) / 16;
    const int G = (int)gridDim.x / (chunks * mgroups);  // workgroups per set
    const int set = (int)blockIdx.x / G;
    const int chunk = SPLIT ? set % chunks : 0;
    const int m0 = 16 * (set / chunks);  // first row of A and C of this group
    const int mrows = min(16, M - m0);
    const int k0 = chunk * kc;
    const int klen = SPLIT ? min(kc, K - k0) : K;
    const uint32_t ldb = (uint32_t)K / 2;           // row stride of B
    const int cpr = klen / 32;                      // 16-byte chunks per row of the range
    const int swz_mask = (cpr % 16 == 0) ? 15 : 0;  // XOR swizzle only when it stays in the row
    const int k_begin = wave * (KSTEPS * 128);      // relative to k0

    const uint32_t lda = VAR == I4I4 ? (uint32_t)K / 2 : (uint32_t)K;  // row stride of A in bytes
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(A, (uint32_t)M * lda);
    const i32x4 rsrc_b = make_rsrc(B, (uint32_t)N * ldb);
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    // DMA of strip s into buffer b: this wave's instructions are KSTEPS
    // consecutive 1 KB pieces of the buffer; lane l of piece j fetches the
    // global chunk stored at buffer position q = 64 j + l.
    uint32_t dma_row_off[KSTEPS];
    bool dma_live[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        const int q = (wave * KSTEPS + t) * 64 + lane;
        const int row = q / cpr, slot = q % cpr;
        dma_live[t] = row < 16;
        dma_row_off[t] = (uint32_t)row * ldb + (uint32_t)k0 / 2 + 16u * (uint32_t)(slot ^ (row & swz_mask));
    }
    auto issue_strip = [&](int s, int b) {
        const uint32_t base = (uint32_t)s * 16u * ldb;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            dma16_nt(rsrc_b, dma_live[t] ? base + dma_row_off[t] : kOutOfRange,
                  lds0 + (uint32_t)b * Cfg::kBufBytes + (uint32_t)(wave * KSTEPS + t) * 1024u);
    };

    // Fragment addresses in a strip buffer: step t reads chunk kc of row r16.
    uint32_t frag_off[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        int col = (k_begin + 128 * t) / 32 + g;
        col = col < cpr ? col : cpr - 1;  // past the range: A is zero there, any in-strip data will do
        frag_off[t] = 16u * (uint32_t)(r16 * cpr + (col ^ (r16 & swz_mask)));
    }

    int s = (int)blockIdx.x - set * G;
    if (s >= strips) return;
    issue_strip(s, 0);

    // A fragments of this wave's K slice (zeros past the range and past M):
    // the 32 k of lane group g as two 16-k MFMA operands, in k order.  They
    // are loaded after the first strip's copies, so the first wait below can
    // leave them in flight: every compute unit reads all of A at once, and
    // the second strip's copies should not wait for that.  kALoads counts
    // these loads (one per step for packed A, two for int8 A).
    // int8 A with WHOLE_A (taken for more than 8 rows): a lane's two
    // operands are bytes 32 g .. 32 g + 31 of a step's 128 for row r16.
    // Loaded that way, consecutive lanes read different rows and every
    // instruction uses half of each 128-byte line it touches; instead each
    // step is loaded as two instructions of 8 rows x 128 bytes in which eight
    // consecutive lanes read one whole line (lane l: row l / 8, plus 8 in the
    // second, 16-byte chunk l % 8), the first wait also waits for A, and the
    // operands are put in place by ds_bpermute once the second strip's copies
    // are out.  With few rows the MFMA-layout loads stay, left in flight by
    // the first wait.
    i32x4 a_lo[KSTEPS], a_hi[KSTEPS];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
        if constexpr (VAR == I4I4) {
            const int kl = k_begin + 128 * j + 32 * g;
            const uint32_t off = kl < klen && r16 < mrows
                                     ? (uint32_t)(m0 + r16) * lda + (uint32_t)(k0 + kl) / 2
                                     : kOutOfRange;
            unpack_chunk<true>(buffer_load16(rsrc_a, off), a_lo[j], a_hi[j]);
        } else if constexpr (WHOLE_A) {
            const int kl = k_begin + 128 * j + 16 * (lane & 7);  // this lane's 16 bytes of the step
            const int row0 = lane >> 3, row1 = 8 + (lane >> 3);
            a_lo[j] = buffer_load16(rsrc_a, kl < klen && row0 < mrows
                                                ? (uint32_t)(m0 + row0) * lda + (uint32_t)(k0 + kl)
                                                : kOutOfRange);
            a_hi[j] = buffer_load16(rsrc_a, kl < klen && row1 < mrows
                                                ? (uint32_t)(m0 + row1) * lda + (uint32_t)(k0 + kl)
                                                : kOutOfRange);
        } else {
            const int kl = k_begin + 128 * j + 32 * g;
            const uint32_t off = kl < klen && r16 < mrows
                                     ? (uint32_t)(m0 + r16) * lda + (uint32_t)(k0 + kl)
                                     : kOutOfRange;
            a_lo[j] = buffer_load16(rsrc_a, off);
            a_hi[j] = buffer_load16(rsrc_a, off == kOutOfRange ? kOutOfRange : off + 16);
        }
    }
    constexpr int kALoads = VAR == I4I4 ? KSTEPS : 2 * KSTEPS;
    // int8 A: from the whole-line layout (a_lo: rows 0-7, a_hi: rows 8-15)
    // to the MFMA operands.  Even lanes of zlo keep a_lo (chunk 2 g' of rows
    // 0-7), odd lanes take a_hi from the even neighbour (the same chunk of
    // rows 8-15); zhi the other way round for the odd chunks; then one
    // bpermute per dword: lane (r16, g) reads lane 8 (r16 % 8) + 2 g, plus
    // 1 for the low operand of rows 8-15 or the high operand of rows 0-7.
    auto place_a = [&]() {
        if constexpr (WHOLE_A) {
            const int up = r16 >> 3;
            const int src_lo = 4 * (8 * (r16 & 7) + 2 * g + up);
            const int src_hi = 4 * (8 * (r16 & 7) + 2 * g + 1 - up);
            const bool odd = (lane & 1) != 0;
            int v_lo[KSTEPS][4], v_hi[KSTEPS][4];
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // quad_perm [1, 0, 3, 2]: each lane takes its neighbour's value
                    const int sw = __builtin_amdgcn_mov_dpp(a_hi[j][d], 0xB1, 0xF, 0xF, false);
                    v_lo[j][d] = __builtin_amdgcn_ds_bpermute(src_lo, odd ? sw : a_lo[j][d]);
                    v_hi[j][d] = __builtin_amdgcn_ds_bpermute(src_hi, odd ? a_lo[j][d] : sw);
                }
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) {
                a_lo[j] = i32x4{v_lo[j][0], v_lo[j][1], v_lo[j][2], v_lo[j][3]};
                a_hi[j] = i32x4{v_hi[j][0], v_hi[j][1], v_hi[j][2], v_hi[j][3]};
            }
        }
    };
    int it = 0;
    int prev = -1;  // strip whose partial tiles await reduction
    // Scales of the strip this wave will reduce next, read one iteration
    // early (the reducing wave of strip s is the wave that reads its scales
    // while strip s is contracted), so the reduction never waits on them.
    float pend_sa = 0.f, pend_sb[4] = {0.f, 0.f, 0.f, 0.f};
    // Integer results are held back: a wave keeps the last sum it reduced and
    // stores it when it reduces the next one, or at the end.  C's small row
    // pieces then reach memory in a burst after the weight stream instead of
    // interleaved with it (interleaved, they slowed the stream measurably).
    // Scaled results are stored at once: their scales are read per strip.
    constexpr bool kHold = OUT == OUT_I32;
    bool held = false;
    int held_n = 0;
    i32x4 held_sum = {0, 0, 0, 0};
    auto put = [&](int n, const i32x4 &sum) {
        if constexpr (SPLIT)
            atomic_add_row4(epi, m0 + r16, N, n, sum);
        else
            store_row4<OUT>(epi, m0 + r16, N, n, sum, pend_sa, pend_sb);
    };
    auto emit = [&](int n, const i32x4 &sum) {
        if (r16 >= mrows) return;
        if (!kHold) {
            put(n, sum);
            return;
        }
        if (held) put(held_n, held_sum);
        held = true;
        held_n = n;
        held_sum = sum;
    };
    for (;;) {
        const int b = it & 1;
        if (it == 0) {
            if constexpr (WHOLE_A)
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): strip s and A, seen by the compiler
            else
                wait_vmcnt<kALoads>();  // this wave's copies of strip s (A's loads are younger)
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();  // strip s is in buffer b; partial tiles of `prev` are in red[b ^ 1]

        // Reduce and store the previous strip (one wave, rotating).
        if (prev >= 0 && wave == (it - 1) % KW) {
            const i32x4 *rp = red + (b ^ 1) * KW * 64;
            i32x4 sum = rp[lane];
#pragma unroll
            for (int w = 1; w < KW; ++w) sum += rp[w * 64 + lane];
            sum >>= kShift;  // the 4-bit operands carried a factor 16 each
            emit(prev * 16 + 4 * g, sum);
        }
        // Next strip's loads into the other buffer (its last readers passed
        // the barrier above).
        const int sn = s + G;
        if (sn < strips) issue_strip(sn, b ^ 1);
        if (it == 0) place_a();  // waits for A, behind the second strip's copies
        if (OUT != OUT_I32 && wave == it % KW && r16 < mrows)
            load_scales<OUT>(epi, m0 + r16, N, s * 16 + 4 * g, pend_sa, pend_sb);

        // Contract this wave's K slice of strip s.
        const uint8_t *buf = smem + b * Cfg::kBufBytes;
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const i32x4 q = *reinterpret_cast<const i32x4 *>(buf + frag_off[t]);
            i32x4 b_lo, b_hi;
            unpack_chunk<true>(q, b_lo, b_hi);
            acc = mfma_16x16x64(b_lo, a_lo[t], acc);
            acc = mfma_16x16x64(b_hi, a_hi[t], acc);
        }
        red[b * KW * 64 + wave * 64 + lane] = acc;
        prev = s;
        ++it;
        if (sn >= strips) break;
        s = sn;
    }
    // The last strip: every partial tile written, then one wave reduces it.
    lds_barrier();
    if (wave == (it - 1) % KW) {
        const i32x4 *rp = red + ((it - 1) & 1) * KW * 64;
        i32x4 sum = rp[lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) sum += rp[w * 64 + lane];
        sum >>= kShift;
        emit(prev * 16 + 4 * g, sum);
    }
    if (kHold && held && r16 < mrows) put(held_n, held_sum);
}

// Several K ranges without atomics (the scaled formats, whose rounded results
// cannot be added): each workgroup contracts every range of its own strips in
// turn (range by range), so no two workgroups share a strip and C needs
// neither a zero fill nor atomic adds.  A of the next range is
// loaded into a second register set while the last strip of the current range
// is contracted; the sums of local strip j (at most KW per workgroup) are
// accumulated across ranges by wave j and stored once, after the last range
// (scaled formats too).  Grid: row groups x workgroups, as for one range.
//
// Requirements (checked on the host): as for gemm_skinny_kernel with SPLIT,
// and at most KW strips per workgroup.
template <int VAR, int KW, int OUT>
__global__ __launch_bounds__(64 * KW) void gemm_skinny_seq_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, Epilogue epi, int M, int N, int K,
    int kc)
{
    static_assert(VAR == W4A8 || VAR == I4I4, "4-bit B with an int8 or int4 A");
    constexpr int KSTEPS = 4;  // ranges are longer than 4096 k
    constexpr int kShift = VAR == I4I4 ? 8 : 4;
    using Cfg = SkinnyCfg<KW, KSTEPS>;
    extern __shared__ __align__(1024) uint8_t smem[];
    i32x4 *red = reinterpret_cast<i32x4 *>(smem + 2 * Cfg::kBufBytes);  // [2][KW][64]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int strips = (N + 15) / 16;
    const int chunks = (K + kc - 1) / kc;
    const int mgroups = (M + 15) / 16;
    const int G = (int)gridDim.x / mgroups;  // workgroups per row group
    const int grp = (int)blockIdx.x / G;
    const int m0 = 16 * grp;
    const int mrows = min(16, M - m0);
    const int s0 = (int)blockIdx.x - grp * G;
    if (s0 >= strips) return;
    const int nloc = (strips - s0 + G - 1) / G;  // this workgroup's strips s0, s0 + G, ...
    const int items = chunks * nloc;             // item i: range i / nloc, local strip i % nloc

    const uint32_t lda = VAR == I4I4 ? (uint32_t)K / 2 : (uint32_t)K;
    const uint32_t ldb = (uint32_t)K / 2;
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(A, (uint32_t)M * lda);
    const i32x4 rsrc_b = make_rsrc(B, (uint32_t)N * ldb);
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    const int k_begin = wave * (KSTEPS * 128);

    auto range_len = [&](int c) { return min(kc, K - c * kc); };
    // This wave's A fragments of range c (zeros past the range and past the group).
    auto load_a = [&](int c, i32x4 (&lo)[KSTEPS], i32x4 (&hi)[KSTEPS]) {
        const int k0 = c * kc, klen = range_len(c);
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
            const int kl = k_begin + 128 * j + 32 * g;
            const bool live = kl < klen && r16 < mrows;
            if constexpr (VAR == I4I4) {
                const uint32_t off = live ? (uint32_t)(m0 + r16) * lda + (uint32_t)(k0 + kl) / 2 : kOutOfRange;
                unpack_chunk<true>(buffer_load16(rsrc_a, off), lo[j], hi[j]);
            } else {
                const uint32_t off = live ? (uint32_t)(m0 + r16) * lda + (uint32_t)(k0 + kl) : kOutOfRange;
                lo[j] = buffer_load16(rsrc_a, off);
                hi[j] = buffer_load16(rsrc_a, live ? off + 16 : kOutOfRange);
            }
        }
    };
    // Copy of range c of strip s into buffer b (layout as in gemm_skinny_kernel).
    auto issue_item = [&](int c, int s, int b) {
        const int cpr = range_len(c) / 32;
        const int swz = (cpr % 16 == 0) ? 15 : 0;
        const uint32_t base = (uint32_t)s * 16u * ldb + (uint32_t)(c * kc) / 2;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const int q = (wave * KSTEPS + t) * 64 + lane;
            const int row = q / cpr, slot = q % cpr;
            const uint32_t off = row < 16 ? base + (uint32_t)row * ldb + 16u * (uint32_t)(slot ^ (row & swz))
                                          : kOutOfRange;
            dma16_nt(rsrc_b, off, lds0 + (uint32_t)b * Cfg::kBufBytes + (uint32_t)(wave * KSTEPS + t) * 1024u);
        }
    };
    auto frag_offsets = [&](int c, uint32_t (&fo)[KSTEPS]) {
        const int cpr = range_len(c) / 32;
        const int swz = (cpr % 16 == 0) ? 15 : 0;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            int col = (k_begin + 128 * t) / 32 + g;
            col = col < cpr ? col : cpr - 1;  // past the range: A is zero there
            fo[t] = 16u * (uint32_t)(r16 * cpr + (col ^ (r16 & swz)));
        }
    };
    i32x4 run = {0, 0, 0, 0};  // wave j: the sum so far of local strip j
    // Wave j adds the partial tiles of item (c, j) to its sum and, after the
    // last range, stores the strip.
    auto reduce = [&](int item, int slot) {
        const int c = item / nloc, j = item - c * nloc;
        if (wave != j) return;
        const i32x4 *rp = red + slot * KW * 64;
#pragma unroll
        for (int w = 0; w < KW; ++w) run += rp[w * 64 + lane];
        if (c == chunks - 1 && r16 < mrows) {
            const int n = (s0 + j * G) * 16 + 4 * g;
            float sa = 0.f, sb[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (OUT != OUT_I32) load_scales<OUT>(epi, m0 + r16, N, n, sa, sb);
            store_row4<OUT>(epi, m0 + r16, N, n, run >> kShift, sa, sb);
        }
    };

    i32x4 a_lo[KSTEPS], a_hi[KSTEPS], n_lo[KSTEPS], n_hi[KSTEPS];
    uint32_t fo[KSTEPS];
    load_a(0, a_lo, a_hi);
    frag_offsets(0, fo);
    issue_item(0, s0, 0);
    for (int i = 0; i < items; ++i) {
        const int b = i & 1;
        const int c = i / nloc;
        wait_vmcnt<0>();
        lds_barrier();  // item i is in buffer b; the partial tiles of item i - 1 in red[b ^ 1]
        if (i > 0) {
            reduce(i - 1, b ^ 1);
            if (c != (i - 1) / nloc) {  // a new range: its A arrived with the wait above
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    a_lo[t] = n_lo[t];
                    a_hi[t] = n_hi[t];
                }
                frag_offsets(c, fo);
            }
        }
        if (i + 1 < items) {
            const int cn = (i + 1) / nloc;
            issue_item(cn, s0 + ((i + 1) - cn * nloc) * G, b ^ 1);
            if (cn != c) load_a(cn, n_lo, n_hi);
        }
        const uint8_t *buf = smem + b * Cfg::kBufBytes;
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const i32x4 q = *reinterpret_cast<const i32x4 *>(buf + fo[t]);
            i32x4 b_lo, b_hi;
            unpack_chunk<true>(q, b_lo, b_hi);
            acc = mfma_16x16x64(b_lo, a_lo[t], acc);
            acc = mfma_16x16x64(b_hi, a_hi[t], acc);
        }
        red[b * KW * 64 + wave * 64 + lane] = acc;
    }
    lds_barrier();  // the last item's partial tiles are written
    reduce(items - 1, (items - 1) & 1);
}

}  // namespace lpgemm
