// Block-sparse products on CDNA4 matrix cores: SDD, DSD and DSTD (the kernel
// template and its launchers).  Included by gemm_br128.hip and
// gemm_br64.hip, which instantiate the launchers for blocks of 128 and of 64
// rows in two translation units compiled side by side; gemm.hip picks one
// by the topology's block height.
//
// George Lin's Blog (MegaBlocks/FlexMoE post):
//  - section 1.2: one block-sparse product replaces the per-expert batched
//    GEMMs; the first layer is SDD (a dense x dense product kept only at the
//    nonzero blocks), then the activation, then DSD (sparse x dense);
//  - section 1.3: 128 x 128 blocks; BCSR walks a block row in order (DSD),
//    the materialised row index gives random access to any block, and the
//    transpose index lists each block column's blocks for DSTD, the weight
//    gradient (sparse^T x dense).
//
// One kernel template serves all three.  A workgroup of 4 wave64s computes
// a 256 x 256 output tile (2 x 2 panels of 128); each wave owns one 128 x 128
// quadrant as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators held in AGPRs
// (fp32 operands: v_mfma_f32_32x32x2_f32), fp32 accumulation:
//   SDD   a pair of block rows of one expert (same column list) x a pair of
//         their nonzero blocks; K = d.  Dual-B (SwiGLU): one block of W1 and
//         the same block of W3 side by side, combined as silu(g) * u.
//   DSD   a pair of block rows x 256 output columns; K walks the rows'
//         blocks (from row_ptr) and their weight rows.  The two-set form
//         (SwiGLU input gradient) walks them twice: the gate projection's
//         blocks against W1, then the up projection's against W3, into one
//         accumulator.
//   DSTD  a pair of block columns x 256 output columns; K walks the
//         columns' blocks (the expert's block rows, from col_ptr) and their
//         dense rows.
// The topology is the block-diagonal one of section 1.3 (each block row
// holds exactly its expert's F column blocks, in order), so the K-block
// indices the transpose and row indices list are closed forms: block row r's
// p-th block is row_ptr[r] + p = r F + p, in column e F + p; block column
// e F + j holds block rows s_e .. s_e + R_e - 1, its p-th block being
// (s_e + p) F + j, where col_ptr[e F + j] = F s_e + j R_e.  The kernels
// compute them instead of reading the lists (row_ptr[r] = r F too), so an
// SDD or DSD tile reads one index entry (its rows' first column block) after
// its row_tiles entry, and a DSTD tile its two col_ptr entries after its
// expert_order entry, before the first operand loads.
//
// Pipeline.  Operand panels go from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of kStages
// stages of 32 KB (K-tile = 64 bytes of K per row), so kStages - 1 K-tiles
// of loads are in flight.  One barrier per K-tile sits in the middle of the
// tile: the MFMAs of the first half run, the barrier publishes the next
// K-tile, and the second half's MFMAs overlap the fragment reads of the
// next K-tile and the issue of the loads kStages - 1 tiles ahead, so the
// matrix cores do not wait on LDS latency at a tile boundary.
//
// LDS layouts.  K-contiguous panels are stored row-major (64-byte rows) with
// an XOR swizzle of the 16-byte chunks and read with ds_read_b128.  Panels
// contiguous along M or N (W1 and W2 in the forward pass, both operands of
// DSTD) are stored k-major and read with ds_read_b64_tr_b16, which hands
// each lane 4 consecutive k of its row: no transpose pass anywhere.
//
// Tile order.  Workgroup ids are remapped so each XCD runs a contiguous
// range of tiles, and the tiles of SDD and DSD go in groups of a few row
// pairs, down the rows first: the tiles that run at the same time on one
// XCD cover a few row pairs x a few column tiles and share both operands'
// panels in that XCD's L2.  DSTD tiles, whose K is the expert's row count,
// go expert by expert in descending size (longest first), in chunks dealt
// to the XCDs in turn.
//
// Last round.  When the tiles do not fill whole rounds of the GPU's compute
// units and the last round would leave most of them idle, an SDD runs that
// round's tiles as two half tiles each (split along M: its activation needs
// the whole K sum), and a DSD given a workspace cuts them into K-segments
// whose fp32 partial sums a second launch adds in segment order
// (dsd_reduce_kernel): the kernel boundary orders the shares before their
// sum, so no workgroup waits on another.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace bsg {

constexpr int kGemmThreads = 256;
constexpr int kRowBytes = 64;                  // K bytes per row and stage
constexpr int kPanelBytes = 128 * kRowBytes;   // 8 KB: 128 rows
constexpr int kSegs = kPanelBytes / 1024;      // 1 KB segments per panel
constexpr int kStageBytes = 4 * kPanelBytes;   // A0 A1 B0 B1
constexpr int kStages = 4;
constexpr int kLdsBytes = kStages * kStageBytes;
// Split DSD tiles: fp32 partial sums of one 256 x 256 tile (256 KB), and at
// most this many K-segments a tile
constexpr int kSplitFloats = kSplitShareBytes / 4;
constexpr int kMaxSplit = 8;
constexpr int kSegsPerWave = kSegs / 4;          // per panel
constexpr int kLoadsPerTile = 4 * kSegsPerWave;  // per wave and K-tile

// Tile order (see xcd_chunked): consecutive DSTD tiles kept on one XCD.
constexpr int kDstdChunk = 8;

template <int DT>
struct Elt;
template <>
struct Elt<kBf16> {
    static constexpr int kKt = 32;  // K per stage
    static constexpr int kBytes = 2;
};
template <>
struct Elt<kF32> {
    static constexpr int kKt = 16;
    static constexpr int kBytes = 4;
};

typedef __attribute__((address_space(3))) char lds_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ------------------------------------------------------------ LDS layouts
//
// K-contiguous panel: 128 rows x 4 chunks of 16 bytes; chunk q of row r at
// slot 4r + (q ^ ((r >> 2) & 3)): the 16 rows one phase of a fragment read
// touches fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kslot(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

// k-major panel: KT rows of 128 M/N values.  bf16: 16 chunks per row, chunk
// q of row k at 16k + (q ^ 4(k & 3)), so the 4 k-rows a transposing read
// touches per 16-lane group use disjoint bank ranges.  fp32: 32 chunks per
// row, unswizzled.
template <int DT>
__device__ __forceinline__ int mnslot(int k, int q) {
    if constexpr (DT == kBf16) return k * 16 + (q ^ ((k & 3) << 2));
    else return k * 32 + q;
}

// Byte offset (from the panel's origin in global memory) of the 16 bytes
// lane `lane` fetches for segment s of a panel; ld = row stride in bytes.
// The swizzle is applied here: lane L lands on byte 16 L of its segment.
template <int DT, bool KC>
__device__ __forceinline__ int64_t seg_offset(int s, int lane, int64_t ld) {
    if constexpr (KC) {  // 16 rows of 64 bytes per segment
        const int row = s * 16 + (lane >> 2);
        const int q = (lane & 3) ^ ((row >> 2) & 3);
        return (int64_t)row * ld + q * 16;
    } else if constexpr (DT == kBf16) {  // 4 k-rows of 256 bytes
        const int k = s * 4 + (lane >> 4);
        const int q = (lane & 15) ^ ((k & 3) << 2);
        return (int64_t)k * ld + q * 16;
    } else {  // fp32: 2 k-rows of 512 bytes
        const int k = s * 2 + (lane >> 5);
        return (int64_t)k * ld + (lane & 31) * 16;
    }
}

// Direct global -> LDS load of 16 bytes per lane: lane L's bytes land at
// LDS byte lds_addr + 16 L (lds_addr is wave-uniform, it goes to M0).  The
// instruction is issued through inline asm in its SGPR-base form (base +
// 32-bit lane offset) so the compiler does not model the LDS write: it would
// otherwise drain every in-flight load (vmcnt(0)) before each LDS read it
// cannot prove disjoint.  The kernel therefore orders these loads itself:
// wait_tiles() below, before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const char* base, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(off), "s"(base)
                 : "memory");
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_u32(const lds_t* p) { return (uint32_t)(uintptr_t)p; }

// -------------------------------------------------------- fragment reads
//
// Lane l of a 32 x 32 x 16 MFMA supplies row (l & 31) of its operand with
// k = 8 (l >> 5) .. + 7 of the current 16.  `r0` is the fragment's first
// row inside the panel, `c` the K-step (16 bf16 / 8 fp32 values).
template <int DT, bool KC>
__device__ __forceinline__ u32x4 frag(const lds_t* panel, int r0, int c) {
    const int lane = threadIdx.x & 63;
    if constexpr (KC) {
        return *(const __attribute__((address_space(3))) u32x4*)(
            panel + kslot(r0 + (lane & 31), 2 * c + (lane >> 5)) * 16);
    } else if constexpr (DT == kBf16) {
        // two transposing reads: within each 16-lane group lane i receives
        // element i % 4 of the 8 bytes fetched by lanes 4j + i / 4 (j = 0..3),
        // so lane i addresses row k0 + i / 4, columns n0 + 4 (i % 4) .. + 3
        const int g = lane >> 4, i = lane & 15;
        const int n = r0 + 16 * (g & 1) + 4 * (i & 3);
        const int k = 16 * c + 8 * (g >> 1) + (i >> 2);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(panel + mnslot<DT>(k, n >> 3) * 16 + (n & 7) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(panel + mnslot<DT>(k + 4, n >> 3) * 16 + (n & 7) * 2));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return u32x4{a[0], a[1], b[0], b[1]};
    } else {
        // fp32 k-major: one element per MFMA step, k = 8c + 4 (l >> 5) + s
        u32x4 v;
        const int m = r0 + (lane & 31);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k = 8 * c + 4 * (lane >> 5) + s;
            v[s] = *(const __attribute__((address_space(3))) uint32_t*)(panel + (k * 128 + m) * 4);
        }
        return v;
    }
}

template <int DT>
__device__ __forceinline__ void mma(f32x16& acc, u32x4 x, u32x4 y);

template <>
__device__ __forceinline__ void mma<kBf16>(f32x16& acc, u32x4 x, u32x4 y) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                  __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
}

// fp32: a 16-byte K chunk holds 4 consecutive k; lane half h of K-step c
// uses k = 8c + 4h + s in step s, for both operands alike.
template <>
__device__ __forceinline__ void mma<kF32>(f32x16& acc, u32x4 x, u32x4 y) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(x[s]), __uint_as_float(y[s]),
                                                   acc, 0, 0, 0);
}

// Wait until at most `tiles` K-tiles of this wave's direct loads are still
// in flight (they retire in issue order); LPT loads per K-tile: 8, or 6 in
// a half tile, which skips the absent M half's panel.
template <int LPT>
__device__ __forceinline__ void wait_tiles(int tiles) {
    static_assert(LPT == 8 || LPT == 6, "8 or 6 loads per K-tile");
    switch (tiles) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPT) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPT) : "memory"); break;
    }
}
static_assert(kLoadsPerTile == 8, "wait_tiles encodes 8 loads per K-tile");
static_assert(kStages <= 4, "wait_tiles covers up to 3 K-tiles in flight behind the waited one");

// ------------------------------------------------------------- epilogue io

template <int OUT>
__device__ __forceinline__ void store4(char* dst, const float* v) {
    if constexpr (OUT == kBf16)
        *(u32x2*)dst = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
        *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
}

template <int OUT>
__device__ __forceinline__ void load4(const char* src, float* v) {
    if constexpr (OUT == kBf16) {
        const u32x2 u = *(const u32x2*)src;
        v[0] = __uint_as_float(u[0] << 16);
        v[1] = __uint_as_float(u[0] & 0xffff0000u);
        v[2] = __uint_as_float(u[1] << 16);
        v[3] = __uint_as_float(u[1] & 0xffff0000u);
    } else {
        const f32x4 f = *(const f32x4*)src;
        v[0] = f[0], v[1] = f[1], v[2] = f[2], v[3] = f[3];
    }
}

// SDD / DSD tile order.  The topology cuts each expert's row tiles (up to
// 256 rows each) into groups of a few (row_tiles entry bits 2-4: the row
// tile's place in its group, bits 5-7: the group's size - 1), so a group
// never spans two experts.  A group's tiles have consecutive ids, down its
// row tiles first: the tiles an XCD runs at once cover a few row tiles of
// one expert x a few column tiles and share both operands' panels.  Tile t
// lies in the group of row tile t / tn, since the groups before it hold
// exactly its first row tile's count of row tiles.
__device__ __forceinline__ void row_tile_of(const int32_t* __restrict__ row_tiles, int tile,
                                              int tn, int& tm, int& tq) {
    const int p0 = tile / tn;
    const int ent = row_tiles[p0];
    const int first = p0 - ((ent >> 2) & 7);
    const int size = ((ent >> 5) & 7) + 1;
    const int local = tile - first * tn;
    tq = local / size;
    tm = first + local % size;
}

// MODE: kModeSdd, kModeSddOne (dual-B SwiGLU: one block per tile),
// kModeDsd, kModeDsd2 (two block sets), kModeDstd.  BK: B operand
// K-contiguous.
// BR: rows of a block, 128 or 64 (bins of 64 rows).  An SDD / DSD tile
// covers up to 256 rows of one expert: Q = 256 / BR consecutive block rows
// ("slots") from block row r0, nq of them present (fewer at the expert's
// end); an absent slot mirrors the last present one (loaded, never stored).
// HALF: a tile with at most 128 rows present.  Its four waves split those
// rows: wave (wm, wn) takes rows 64 wm .. 64 wm + 63 x the 128 columns of N
// half wn, as 2 x 4 accumulators, and the absent half's panel is not loaded
// (6 direct loads per K-tile instead of 8).
// tile: the SDD / DSD tile in group order (DSTD maps its own).  seg of nseg:
// for a split DSD tile, the share of its K-blocks to sum, written to `part`
// (fp32, no epilogue); for a split SDD row tile (nseg = 2, HALF), which half
// of its block rows to run.  Unsplit: 0 of 1, part NULL.
template <int DT, int MODE, bool BK, int EPI, int OUT, bool SWAP, bool HALF, int BR>
__device__ __forceinline__ void gemm_tile(const GemmParams& P, char* smem, int tile, int seg,
                                          int nseg, float* part) {
    constexpr int ES = Elt<DT>::kBytes;
    constexpr int KT = Elt<DT>::kKt;
    static_assert(BR == 128 || BR == 64, "blocks of 128 or 64 rows");
    constexpr int QB = kBlock / BR;                       // slots per 128-row panel
    constexpr int KPB = (MODE == kModeDstd ? BR : kBlock) / KT;  // K-tiles per K-block
    constexpr int OES = OUT == kBf16 ? 2 : 4;
    constexpr bool AK = MODE != kModeDstd;
    constexpr bool DUAL = EPI == kEpiSiluMul || EPI == kEpiSiluMulSave;
    constexpr bool SDD = MODE == kModeSdd || MODE == kModeSddOne;
    constexpr bool DSD = MODE == kModeDsd || MODE == kModeDsd2;
    constexpr bool SPLIT = MODE != kModeDstd;  // loads of a K-tile over two half-steps
    static_assert(KT / (DT == kBf16 ? 16 : 8) == 2, "two MFMA K-steps per K-tile");
    static_assert(!HALF || ((SDD && !DUAL) || DSD) && SWAP, "half tiles: SDD / DSD, row-major C");
    constexpr int LPT = HALF ? kLoadsPerTile - 2 : kLoadsPerTile;  // direct loads per K-tile
    constexpr int NH = HALF ? 1 : 2;      // 64-row output halves per wave
    constexpr int NMI = HALF ? 2 : 4;     // 32-row A fragments per wave
    lds_t* lds = (lds_t*)smem;

    // ---- the tile: SDD / DSD, `tile` in the group order (the launch's
    // wrapper maps workgroups to tiles); DSTD, from the workgroup index here
    const int F = P.F;
    const int tn = MODE == kModeSdd ? (F + 1) / 2 : MODE == kModeSddOne ? F : P.ntn;
    // tm: row pair (SDD / DSD) or expert column pair (DSTD); tq: N tile
    int tm, tq;
    if constexpr (MODE == kModeDstd) {
        // a DSTD tile's K is its expert's rows: experts longest first, each
        // expert's tiles in groups of column pairs x N tiles
        const int ntiles = P.E * ((F + 1) / 2) * tn;
        if ((int)blockIdx.x >= ntiles) return;
        const int cpe = (F + 1) / 2, per_e = cpe * tn;
        const int t = xcd_chunked(blockIdx.x, ntiles, kDstdChunk);
        const int rank = t / per_e;
        int j;
        grouped_tile(t - rank * per_e, cpe, tn, P.group, j, tq);
        tm = P.expert_order[rank] * cpe + j;
    } else {
        row_tile_of(P.row_tiles, tile, tn, tm, tq);
    }

    // the wave index is uniform: keep it (and every LDS stage address derived
    // from it) in scalar registers
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lh = lane >> 5;
    // first row of this wave's output inside its block row (half tiles)
    const int roff = HALF ? 64 * wm : 0;

    // ---- the tile's two M halves: SDD / DSD, the rows of slots 0 .. Q - 1;
    // DSTD, a pair of block columns (an absent second mirrors the first)
    int r0 = 0, nq = 1;        // SDD / DSD: first block row, slots present
    int mrow0 = 0, mrow1 = 0;  // DSTD: the two block columns
    bool m1;                   // second M half present
    if constexpr (MODE == kModeDstd) {
        const int cpe = (F + 1) / 2;
        const int e = tm / cpe, j = tm % cpe;
        mrow0 = e * F + 2 * j;
        m1 = 2 * j + 1 < F;
        mrow1 = m1 ? mrow0 + 1 : mrow0;
    } else {
        const int ent = P.row_tiles[tm];
        r0 = ent >> 8;
        nq = (ent & 3) + 1;
        if constexpr (SDD) {
            // a row tile of the SDD's split last round: half seg of it (its
            // first QB block rows, or the rest)
            if (nseg == 2) {
                r0 += seg * QB;
                nq = seg == 0 ? min(nq, QB) : nq - QB;
            }
        }
        m1 = nq > QB;
    }
    // first block of each slot's block row (an absent slot: the last present
    // one): every block row holds its expert's F blocks, so row_ptr[r] = r F
    int rps[2 * QB];
    if constexpr (SDD || DSD) {
#pragma unroll
        for (int i = 0; i < 2 * QB; ++i) rps[i] = (r0 + min(i, nq - 1)) * F;
    }
    // the slot of the A rows this wave loads into panel p (each wave loads
    // 32 consecutive rows of a panel, so they lie in one slot)
    auto aslot = [&](int pnl) { return QB * pnl + (QB == 2 ? (wave >> 1) : 0); };
    // ---- N halves
    bool n1;
    int bcol0 = 0, bcol1 = 0;  // SDD: column blocks of B
    const int rp0 = (SDD || DSD) ? rps[0] : 0;  // the slots share this column list
    // the rows' first column block, e F (the tile's one index load): their
    // p-th block lies in column block e F + p
    const int cb0 = (SDD || DSD) ? P.col_idx[rp0] : 0;
    if constexpr (MODE == kModeSdd) {
        n1 = 2 * tq + 1 < F;
        bcol0 = cb0 + 2 * tq;
        bcol1 = n1 ? bcol0 + 1 : bcol0;
    } else if constexpr (MODE == kModeSddOne) {
        n1 = DUAL;
        bcol0 = bcol1 = cb0 + tq;
    } else {
        n1 = tq * 256 + 128 < P.N;
    }
    const int64_t n0 = (int64_t)tq * 256;
    const int64_t n1off = n1 ? 128 : 0;  // an absent N half mirrors half 0

    // ---- K extent in K-blocks (DSD / DSTD; the two-set DSD walks the row's
    // blocks twice, first in set one, then in set two), and what a DSTD
    // tile's K-block indices follow from: its expert's first block row s_e
    // and the two columns' places j0, j1 in the expert (a DSD tile's follow
    // from rp0 and cb0)
    int nblk = 0, rowlen = 0, se = 0, j0 = 0, j1 = 0;
    if constexpr (DSD) {
        rowlen = F;
        nblk = MODE == kModeDsd2 ? 2 * rowlen : rowlen;
    } else if constexpr (MODE == kModeDstd) {
        const int cp0 = P.col_ptr[mrow0];
        nblk = P.col_ptr[mrow0 + 1] - cp0;  // R_e
        const int e = mrow0 / F;
        j0 = mrow0 - e * F;
        j1 = mrow1 - e * F;
        se = (cp0 - j0 * nblk) / F;  // col_ptr[e F + j] = F s_e + j R_e
    }

    // ---- per-lane load offsets (constant over K)
    const int64_t lda_b = (SDD ? P.lda : kBlock) * ES;  // A row (or k-row) stride
    const int64_t ldb_b = P.ldb * ES;
    uint32_t aoff[kSegsPerWave], boff[kSegsPerWave];
#pragma unroll
    for (int j = 0; j < kSegsPerWave; ++j) {
        const int s = wave * kSegsPerWave + j;
        // rows contiguous along K (SDD, DSD) are addressed inside their slot
        aoff[j] = (uint32_t)seg_offset<DT, AK>(AK ? s % (BR / 16) : s, lane, lda_b);
        boff[j] = (uint32_t)seg_offset<DT, BK>(s, lane, ldb_b);
    }
    // DSD: this wave's A block in panel p is slot 0's block plus dA[p]
    int dA[2] = {0, 0};
    if constexpr (DSD) {
#pragma unroll
        for (int pnl = 0; pnl < 2; ++pnl) dA[pnl] = rps[aslot(pnl)] - rps[0];
    }
    // uniform global origins of the four panels of K-tile t
    struct Bases {
        const char *a0, *a1, *b0, *b1;
    };
    // the K-block indices of K-tile t (DSD / DSTD; K-blocks from kb0 on): the
    // block of each M half and its dense row block (DSD: weight row block,
    // kSecondSet marking the second set of the two-set form)
    struct TIdx {
        int b0, b1, row;
    };
    int kb0 = 0;
    auto tidx = [&](int t) -> TIdx {
        TIdx r{0, 0, 0};
        if constexpr (DSD) {
            int p = kb0 + t / KPB;
            int set = 0;
            if (MODE == kModeDsd2 && p >= rowlen) {
                p -= rowlen;
                set = kSecondSet;
            }
            r.b0 = rp0 + p + dA[0];
            r.b1 = rp0 + p + dA[1];
            r.row = (cb0 + p) | set;
        } else if constexpr (MODE == kModeDstd) {
            const int p = kb0 + t / KPB;
            r.b0 = (se + p) * F + j0;
            r.b1 = (se + p) * F + j1;
            r.row = se + p;
        }
        return r;
    };
    auto bases = [&](int t, const TIdx& ti) -> Bases {
        Bases r;
        const int koff = (t % KPB) * KT;
        if constexpr (SDD) {
            const char* A = (const char*)P.a + (int64_t)t * KT * ES;
            r.a0 = A + (int64_t)BR * (r0 + min(aslot(0), nq - 1)) * P.lda * ES;
            r.a1 = A + (int64_t)BR * (r0 + min(aslot(1), nq - 1)) * P.lda * ES;
            const char* B1 = DUAL ? (const char*)P.b2 : (const char*)P.b;
            if constexpr (BK) {
                r.b0 = (const char*)P.b + ((int64_t)kBlock * bcol0 * P.ldb + (int64_t)t * KT) * ES;
                r.b1 = B1 + ((int64_t)kBlock * bcol1 * P.ldb + (int64_t)t * KT) * ES;
            } else {
                r.b0 = (const char*)P.b + ((int64_t)t * KT * P.ldb + (int64_t)kBlock * bcol0) * ES;
                r.b1 = B1 + ((int64_t)t * KT * P.ldb + (int64_t)kBlock * bcol1) * ES;
            }
        } else {
            const int blk0 = __builtin_amdgcn_readfirstlane(ti.b0);
            const int blk1 = __builtin_amdgcn_readfirstlane(ti.b1);
            int rowb = __builtin_amdgcn_readfirstlane(ti.row);
            if constexpr (DSD) {
                const char* As = (const char*)P.a;
                const char* Bs = (const char*)P.b;
                if constexpr (MODE == kModeDsd2) {
                    if (rowb & kSecondSet) {  // uniform: the K-block is in set two
                        As = (const char*)P.a2;
                        Bs = (const char*)P.b2;
                        rowb &= ~kSecondSet;
                    }
                }
                r.a0 = As + ((int64_t)blk0 * BR * kBlock + koff) * ES;
                r.a1 = As + ((int64_t)blk1 * BR * kBlock + koff) * ES;
                const int64_t krow = (int64_t)kBlock * rowb + koff;
                if constexpr (BK) {
                    r.b0 = Bs + (n0 * P.ldb + krow) * ES;
                    r.b1 = r.b0 + n1off * P.ldb * ES;
                } else {
                    r.b0 = Bs + (krow * P.ldb + n0) * ES;
                    r.b1 = r.b0 + n1off * ES;
                }
            } else {  // DSTD: A = block^T (k-major as stored), B = dense rows
                r.a0 = (const char*)P.a + ((int64_t)blk0 * BR * kBlock + (int64_t)koff * kBlock) * ES;
                r.a1 = (const char*)P.a + ((int64_t)blk1 * BR * kBlock + (int64_t)koff * kBlock) * ES;
                const int64_t drow = (int64_t)BR * rowb + koff;
                r.b0 = (const char*)P.b + (drow * P.ldb + n0) * ES;
                r.b1 = r.b0 + n1off * ES;
            }
        }
        r.a0 = uniform_ptr(r.a0);
        r.a1 = uniform_ptr(r.a1);
        r.b0 = uniform_ptr(r.b0);
        r.b1 = uniform_ptr(r.b1);
        return r;
    };
    // load j (0..7) of K-tile t into its stage: panel j & 3, segment j >> 2
    const uint32_t lds0 = lds_u32(lds) + wave * kSegsPerWave * 1024;
    auto dma = [&](int t, const Bases& b, int j) {
        const int pnl = j & 3, sg = j >> 2;
        if (HALF && pnl == 1) return;  // the absent M half
        const uint32_t dst = lds0 + (t % kStages) * kStageBytes + pnl * kPanelBytes + sg * 1024;
        const char* base = pnl == 0 ? b.a0 : pnl == 1 ? b.a1 : pnl == 2 ? b.b0 : b.b1;
        dma16(dst, base, pnl < 2 ? aoff[sg] : boff[sg]);
    };

    // ---- this wave's output: does it exist; per 64-row half h of it, the
    // tile row it starts at, its slot, whether the slot is present and (SDD)
    // its output block and first row inside that block
    const bool active =
        (HALF ? (64 * wm) / BR < nq : (wm == 0 || m1)) && (DUAL || wn == 0 || n1);
    const int mrow = wm ? mrow1 : mrow0;  // DSTD: this wave's block column
    auto hrow = [&](int h) { return HALF ? 64 * wm : 128 * wm + 64 * h; };
    auto hslot = [&](int h) { return hrow(h) / BR; };
    auto hpresent = [&](int h) { return MODE == kModeDstd || hslot(h) < nq; };
    auto hin = [&](int h) { return hrow(h) % BR; };
    auto hblk = [&](int h) -> int {
        if constexpr (MODE == kModeSdd) return rps[hslot(h)] + 2 * tq + wn;
        else if constexpr (MODE == kModeSddOne) return rps[hslot(h)] + tq;
        else return 0;
    };
    constexpr int NI = DUAL ? 2 : 4;

    // Backward epilogues (bf16): the saved factors, read one 32-row slab ahead
    // of their use so the loads of slab mi + 1 overlap the work on slab mi;
    // with one plane, slab 0 is requested before the last K-tile (two planes
    // in flight there would not fit the registers).
    // GeLU: one plane (the derivative); SwiGLU: two (silu(g), u * silu'(g)).
    // (The two-plane prefetch does not fit beside the registers of a B
    // operand read as stored; that variant reads the factors at use.)
    constexpr bool TWO_IN = EPI == kEpiSiluMulBwd;
    constexpr bool PRE = TWO_IN && BK && OUT == kBf16;
    // GeLU backward (bf16): the saved derivative goes straight into LDS with
    // direct loads, 32-row slabs of the wave's block (8 KB each, whole
    // 256-byte rows, so every load covers whole lines), and is read back in
    // the accumulator layout.  Slab 0 lands in a per-wave 8 KB buffer past the
    // ring, requested before the last K-tile; slabs 1 and 2 in the upper half
    // of the wave's staging region once the ring is free; slab 3 in the
    // buffer again once slab 0 has been read.
    constexpr bool GLDS = EPI == kEpiGeluBwd && OUT == kBf16;
    u32x2 hsave[2][NI][4];
    u32x2 qsave[TWO_IN ? 2 : 1][NI][4];
    auto hload = [&](int mi, int buf) {
        const int h = HALF ? 0 : mi >> 1;
        const int64_t base =
            (int64_t)hblk(h) * BR * kBlock + (hin(h) + 32 * (mi & 1) + l32) * kBlock;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nloc = 32 * ni + 8 * g + 4 * lh;
                const int64_t off = base + nloc;
                hsave[buf][ni][g] = *(const u32x2*)((const char*)P.aux_in + off * 2);
                if constexpr (TWO_IN)
                    qsave[buf][ni][g] = *(const u32x2*)((const char*)P.aux_in + (P.plane + off) * 2);
            }
    };

    // direct loads of derivative slab `sl` (rows 32 sl .. + 31 of this wave's
    // rows, one 128-column block) into an 8 KB LDS buffer, row r at 256 r with
    // its 16-byte chunk c at slot c ^ (r & 15), the layout the epilogue's
    // staging uses; 8 loads, each 4 rows
    auto gslab = [&](int sl, uint32_t dst) {
        const int hh = HALF ? 0 : sl >> 1;
        const char* src = uniform_ptr((const char*)P.aux_in +
                                      ((int64_t)hblk(hh) * BR * kBlock +
                                       (int64_t)(hin(hh) + 32 * (sl & 1)) * kBlock) * 2);
        const int rr = lane >> 4;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + rr;
            dma16(dst + j * 1024, src, (uint32_t)(r * 256 + (((lane & 15) ^ (r & 15)) << 4)));
        }
    };
    const uint32_t gbuf = lds_u32(lds) + kLdsBytes + wave * 8192;  // slabs 0 and 3

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // rows of this wave's fragments inside its panels
    int bpanel[4], brow[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        if constexpr (DUAL) {  // gate columns in sub-tiles 0,1 (panel B0), up in 2,3 (B1)
            bpanel[ni] = 2 + (ni < 2 ? 0 : 1);
            brow[ni] = wn * 64 + 32 * (ni & 1);
        } else {
            bpanel[ni] = 2 + wn;
            brow[ni] = 32 * ni;
        }
    }
    // fragment g of K-step c of K-tile t: g < 4 -> A row tile g, else B tile g - 4
    auto read1 = [&](int t, int c, int g, u32x4* af, u32x4* bf) {
        const lds_t* st = lds + (t % kStages) * kStageBytes;
        if (HALF && g < 4) {  // rows 64 wm .. + 63 of the one A panel
            if (g < NMI) af[g] = frag<DT, AK>(st, roff + 32 * g, c);
        } else if (g < 4) {
            af[g] = frag<DT, AK>(st + wm * kPanelBytes, 32 * g, c);
        } else {
            bf[g - 4] = frag<DT, BK>(st + bpanel[g - 4] * kPanelBytes, brow[g - 4], c);
        }
    };
    auto mma2 = [&](int g, const u32x4* af, const u32x4* bf) {
        if (2 * g >= 4 * NMI) return;  // half tiles: A fragments 0, 1 only
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mi = (2 * g + h) >> 2, ni = (2 * g + h) & 3;
            if constexpr (SWAP) mma<DT>(acc[mi][ni], bf[ni], af[mi]);
            else mma<DT>(acc[mi][ni], af[mi], bf[ni]);
        }
    };

    // ---- main loop, software pipelined; every wave runs the MFMAs (also a
    // wave whose half of a half tile is absent: stale data, nothing stored),
    // so no branch ever sits around the accumulators.
    //   first half : 16 MFMAs of K-step 0, interleaved with the fragment
    //                reads of K-step 1 (same K-tile)
    //   publish    : wait for K-tile kt + 1's loads, barrier (past it, every
    //                wave holds K-tile kt's fragments: its stage is free)
    //   second half: 16 MFMAs of K-step 1, interleaved with the fragment
    //                reads of K-step 0 of K-tile kt + 1 and the loads of
    //                K-tile kt + kStages into K-tile kt's stage
    // SDD and DSD issue those 8 loads half in this second half and half in
    // the next first half, one every other MFMA pair, so the address unit
    // never takes a burst of 8 from every wave at once (measured 2-5 %
    // faster for them; DSTD keeps all 8 in the second half, where the split
    // measured slower).
    u32x4 a0f[4], b0f[4], a1f[4], b1f[4];
    TIdx nti{0, 0, 0};  // indices of the next K-tile to load
    Bases pend{};       // K-tile whose loads 4..7 the next first half issues
    auto first_half = [&](int kt, int nk) {
        const bool rest = SPLIT && kt >= 1 && kt + kStages - 1 < nk;
        if (kt + kStages < nk) nti = tidx(kt + kStages);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            read1(kt, 1, g, a1f, b1f);
            if (rest && (g & 1)) dma(kt + kStages - 1, pend, 4 + (g >> 1));
            mma2(g, a0f, b0f);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto second_half = [&](int kt, bool publish, bool load) {
        if (publish) {
            if (load) pend = bases(kt + kStages, nti);
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                read1(kt + 1, 0, g, a0f, b0f);
                if (load && (!SPLIT || (g & 1))) dma(kt + kStages, pend, SPLIT ? g >> 1 : g);
                mma2(g, a1f, b1f);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int g = 0; g < 8; ++g) mma2(g, a1f, b1f);
        }
    };
    auto run = [&](int nk) {
        if (nk <= 0) return;
        for (int t = 0; t < kStages && t < nk; ++t) {
            const Bases b = bases(t, tidx(t));
#pragma unroll
            for (int j = 0; j < kLoadsPerTile; ++j) dma(t, b, j);
        }
        wait_tiles<LPT>(min(kStages - 1, nk - 1));
        __syncthreads();
#pragma unroll
        for (int g = 0; g < 8; ++g) read1(0, 0, g, a0f, b0f);
        int kt = 0;
        // steady state: publish K-tile kt + 1, load K-tile kt + kStages
        for (; kt + kStages < nk; ++kt) {
            first_half(kt, nk);
            wait_tiles<LPT>(kStages - 2);
            __syncthreads();
            second_half(kt, true, true);
        }
        // tail: publish without new loads
        for (; kt + 1 < nk; ++kt) {
            first_half(kt, nk);
            wait_tiles<LPT>(min(kStages - 2, nk - 2 - kt));
            __syncthreads();
            second_half(kt, true, false);
        }
        // last K-tile (every direct load has landed: the counter holds only
        // what the epilogue's prefetch adds)
        if constexpr (GLDS) {
            if (active) gslab(0, gbuf);
        }
        first_half(kt, nk);
        second_half(kt, false, false);
    };

    if constexpr (SDD) {
        run(P.K / KT);
    } else {
        // the tile's K-blocks (segment seg of nseg: a split tile's share)
        kb0 = (int)((int64_t)seg * nblk / nseg);
        const int kb1 = (int)((int64_t)(seg + 1) * nblk / nseg);
        run((kb1 - kb0) * KPB);
    }

    // ---- a split tile's share (DSD): its fp32 partial sums go to `part` in
    // the accumulator layout (per wave, per 32 x 32 block, 16 values a lane,
    // 4 KB contiguous); the reduction launch adds the shares in segment order
    if constexpr (DSD) {
        if (part) {
            float* wp = part + wave * (kSplitFloats / 4) + lane * 16;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(f32x4*)(wp + (mi * 4 + ni) * 1024 + 4 * q) =
                            f32x4{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1],
                                  acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]};
            return;
        }
    }

    // ---- epilogue.  bf16 results go out through LDS: each
    // wave writes half of its 128 x 128 quarter (64 rows) at a time into a
    // private 32 KB region in the accumulator layout, then reads it back row
    // by row, so every store instruction writes 4 whole 256-byte rows
    // (16 contiguous bytes a lane), non-temporal, so the results do not
    // evict operand panels that other workgroups still read from the L2
    // (4-7 % faster at MoE-Small sizes).  Epilogues with two outputs stage them
    // side by side: GeLU with the derivative kept (derivative, then
    // activation) and the SwiGLU backward (gate, then up projection).
    constexpr bool STAGE = OUT == kBf16;
    if constexpr (STAGE) __syncthreads();  // every wave is done with the operand ring
    if (!active) return;
    if constexpr (PRE) hload(0, 0);

    // staging: row r (256 bytes) of a 64-row sub-region holds 16 chunks of
    // 16 bytes, chunk c at slot c ^ (r & 15), so the 16 lanes reading one row
    // and the 16 rows one accumulator write touches both spread over all banks
    lds_t* region = lds + wave * (kLdsBytes / 4);
    if constexpr (GLDS) {
        gslab(1, lds_u32(region) + 16384);
        if constexpr (NMI > 2) gslab(2, lds_u32(region) + 24576);
    }
    // the LDS buffer that holds derivative slab sl
    auto gsrc = [&](int sl) -> const lds_t* {
        return sl == 1 ? region + 16384 : sl == 2 ? region + 24576 : lds + kLdsBytes + wave * 8192;
    };
    // wait until slab mi has landed.  Direct loads and stores retire in issue
    // order; in flight behind slab mi: full tiles, slabs 1 and 2 behind 0,
    // slab 2 behind 1, slab 3 and half 0's 16 stores behind 2, the stores
    // behind 3; half tiles, slab 1 behind 0
    auto gwait = [&](int mi) {
        if constexpr (NMI > 2) {
            if (mi == 0) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            else if (mi == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else if (mi == 2) {
                if (hpresent(0)) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            } else {
                if (hpresent(0)) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        } else {
            if (mi == 0) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    };
    auto stage_put = [&](lds_t* sub, int mi, int ni, int g, const float* v) {
        const int row = (SWAP ? 32 * mi : 32 * ni) % 64 + l32;
        const int chunk = SWAP ? 4 * ni + g : 4 * mi + g;
        *(__attribute__((address_space(3))) u32x2*)(sub + row * 256 +
                                                      ((chunk ^ (row & 15)) << 4) + lh * 8) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    };
    // dual B (SwiGLU): a wave's slice is 64 columns, so a staged row is 128
    // bytes (8 chunks, chunk c at slot c ^ (r & 7)), and a store instruction
    // writes 8 rows of 128 contiguous bytes
    auto stage_put_d = [&](lds_t* sub, int mi, int ni, int g, const float* v) {
        const int row = (32 * mi) % 64 + l32;
        const int chunk = 4 * ni + g;
        *(__attribute__((address_space(3))) u32x2*)(sub + row * 128 +
                                                      ((chunk ^ (row & 7)) << 4) + lh * 8) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    };
    auto stage_flush_d = [&](const lds_t* sub, char* base) {  // base: the half's row 0
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int chunk = lane & 7;
#pragma unroll 4
        for (int rr = 0; rr < 8; ++rr) {
            const int row = 8 * rr + (lane >> 3);
            const u32x4 u = *(const __attribute__((address_space(3))) u32x4*)(
                sub + row * 128 + ((chunk ^ (row & 7)) << 4));
            __builtin_nontemporal_store(u, (u32x4*)(base + row * (kBlock * 2) + chunk * 16));
        }
    };
    auto stage_flush = [&](const lds_t* sub, char* base, int64_t row_bytes) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int chunk = lane & 15;
#pragma unroll 4
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 4 * rr + (lane >> 4);
            const u32x4 u = *(const __attribute__((address_space(3))) u32x4*)(
                sub + row * 256 + ((chunk ^ (row & 15)) << 4));
            __builtin_nontemporal_store(u, (u32x4*)(base + row * row_bytes + chunk * 16));
        }
    };
    // top-1 DSD: the staged rows also go to token order, y[t] = rd(g_t * v)
    // with v the row as stored (the combine of one pick, bit for bit).  Lane
    // l holds the assignment and gate of row l of each 64-row half, read once
    // here; the flush takes them by lane shuffle.
    int sc_a[2] = {-1, -1};
    float sc_g[2] = {1.0f, 1.0f};
    if constexpr (EPI == kEpiScatter) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
            sc_a[h] = hpresent(h) ? P.scat_rows[(int64_t)BR * r0 + hrow(h) + lane] : -1;
        if (P.scat_gate) {
#pragma unroll
            for (int h = 0; h < NH; ++h) sc_g[h] = sc_a[h] >= 0 ? P.scat_gate[sc_a[h]] : 1.0f;
        }
    }
    // Eight rows a batch: every shuffle and LDS read of the batch is issued
    // before the first store, so their latencies overlap instead of adding up
    // row by row (the stores sit under a per-row mask: pad rows go nowhere).
    auto scatter_flush = [&](const lds_t* sub, int h) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int chunk = lane & 15;
        const int64_t col = n0 + wn * 128 + chunk * 8;
#pragma unroll
        for (int r8 = 0; r8 < 16; r8 += 8) {
            int a[8];
            float g[8];
            u32x4 u[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 4 * (r8 + i) + (lane >> 4);
                a[i] = __shfl(sc_a[h], row, kWave);
                g[i] = __shfl(sc_g[h], row, kWave);
                u[i] = *(const __attribute__((address_space(3))) u32x4*)(
                    sub + row * 256 + ((chunk ^ (row & 15)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x4 o = u[i];
                if (P.scat_gate) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o[j] = pack_bf16x2(g[i] * __uint_as_float(u[i][j] << 16),
                                           g[i] * __uint_as_float(u[i][j] & 0xffff0000u));
                }
                if (a[i] >= 0)
                    __builtin_nontemporal_store(
                        o, (u32x4*)((char*)P.scat_out + ((int64_t)a[i] * P.scat_ld + col) * 2));
            }
        }
    };
    // origin of half h of this wave's quarter in the output, and the row
    // pitch (bytes)
    const int64_t orow = (SDD ? kBlock : P.ldc) * OES;
    auto hbase = [&](int h) -> char* {
        if constexpr (SDD)
            return (char*)P.out + ((int64_t)hblk(h) * BR * kBlock + hin(h) * kBlock) * OES;
        else if constexpr (MODE == kModeDstd && SWAP)
            return (char*)P.out +
                   (((int64_t)kBlock * mrow + 64 * h) * P.ldc + n0 + wn * 128) * OES;
        else if constexpr (SWAP)
            return (char*)P.out + (((int64_t)BR * r0 + hrow(h)) * P.ldc + n0 + wn * 128) * OES;
        else
            return (char*)P.out + ((n0 + wn * 128 + 64 * h) * P.ldc + (int64_t)kBlock * mrow) * OES;
    };

    auto unpack = [](u32x2 u, float* f) {
        f[0] = __uint_as_float(u[0] << 16);
        f[1] = __uint_as_float(u[0] & 0xffff0000u);
        f[2] = __uint_as_float(u[1] << 16);
        f[3] = __uint_as_float(u[1] & 0xffff0000u);
    };

    // two halves of 64 staging rows: M slabs (mi) 2h, 2h + 1 with a
    // row-major output, N slabs (ni) 2h, 2h + 1 with the transposed one
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int b = 0; b < (SWAP ? NI : 4); ++b) {
                const int mi = SWAP || !STAGE ? 2 * h + a : b;
                const int ni = SWAP || !STAGE ? b : 2 * h + a;
                if constexpr (PRE) {
                    if (b == 0 && mi + 1 < NMI) hload(mi + 1, (mi + 1) & 1);
                }
                if constexpr (GLDS) {
                    if (b == 0) gwait(mi);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) v[s] = acc[mi][ni][4 * g + s];
                    if constexpr (SDD) {
                        // block-major output: (m, n) of block b at b*BR*128 + m*128 + n
                        const int hh = HALF ? 0 : mi >> 1;
                        const int m = hin(hh) + 32 * (mi & 1) + l32;
                        const int nloc = DUAL ? wn * 64 + 32 * ni + 8 * g + 4 * lh
                                              : 32 * ni + 8 * g + 4 * lh;
                        const int64_t off = (int64_t)hblk(hh) * BR * kBlock + m * kBlock + nloc;
                        const bool here = hpresent(hh);
                        if constexpr (EPI == kEpiSiluMul) {
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                v[s] = silu_f(v[s]) * acc[mi][ni + 2][4 * g + s];
                        } else if constexpr (EPI == kEpiSiluMulSave) {
                            // A = silu(g) u, and for the backward silu(g) and u silu'(g)
                            float sv[4], qv[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const float u = acc[mi][ni + 2][4 * g + s];
                                float sp;
                                silu_and_grad(v[s], sv[s], sp);
                                qv[s] = u * sp;
                                v[s] = sv[s] * u;
                            }
                            if constexpr (STAGE) {
                                stage_put_d(region + 8192, mi, ni, g, sv);
                                stage_put_d(region + 16384, mi, ni, g, qv);
                            } else if (here) {
                                store4<OUT>((char*)P.aux_out + off * OES, sv);
                                store4<OUT>((char*)P.aux_out + (P.plane + off) * OES, qv);
                            }
                        } else if constexpr (EPI == kEpiGelu) {
#pragma unroll
                            for (int s = 0; s < 4; ++s) v[s] = gelu_f(v[s]);
                        } else if constexpr (EPI == kEpiGeluSave) {
                            // the activation and, for the backward, its derivative
                            float gp[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s) gelu_and_grad(v[s], v[s], gp[s]);
                            if constexpr (STAGE) stage_put(region, mi, ni, g, gp);
                            else if (here) store4<OUT>((char*)P.aux_out + off * OES, gp);
                        } else if constexpr (EPI == kEpiGeluBwd) {
                            // dH = dA * GeLU'(h), the derivative saved by the forward
                            float gv[4];
                            if constexpr (GLDS)
                                unpack(*(const __attribute__((address_space(3))) u32x2*)(
                                           gsrc(mi) + l32 * 256 +
                                           (((4 * ni + g) ^ (l32 & 15)) << 4) + lh * 8),
                                       gv);
                            else
                                load4<OUT>((const char*)P.aux_in + off * OES, gv);
#pragma unroll
                            for (int s = 0; s < 4; ++s) v[s] *= gv[s];
                        } else if constexpr (EPI == kEpiSiluMulBwd) {
                            // gate projection dA * u silu'(g) (plane 0 of the
                            // output), up projection dA * silu(g) (plane 1)
                            float sv[4], qv[4], up[4];
                            if constexpr (PRE) {
                                unpack(hsave[mi & 1][ni][g], sv);
                                unpack(qsave[mi & 1][ni][g], qv);
                            } else {
                                load4<OUT>((const char*)P.aux_in + off * OES, sv);
                                load4<OUT>((const char*)P.aux_in + (P.plane + off) * OES, qv);
                            }
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                up[s] = v[s] * sv[s];
                                v[s] *= qv[s];
                            }
                            if constexpr (STAGE) stage_put(region + 16384, mi, ni, g, up);
                            else if (here) store4<OUT>((char*)P.out + (P.plane + off) * OES, up);
                        }
                        if constexpr (STAGE && DUAL) {
                            stage_put_d(region, mi, ni, g, v);
                        } else if constexpr (STAGE) {
                            stage_put(EPI == kEpiGeluSave ? region + 16384 : region, mi, ni, g, v);
                        } else if (here) {
                            store4<OUT>((char*)P.out + off * OES, v);
                        }
                    } else if constexpr (STAGE) {
                        stage_put(region, mi, ni, g, v);
                    } else if constexpr (SWAP) {  // DSD, or DSTD with row-major C
                        const int hh = HALF ? 0 : mi >> 1;
                        const int64_t row = MODE == kModeDstd
                                                ? (int64_t)kBlock * mrow + 32 * mi + l32
                                                : (int64_t)BR * r0 + hrow(hh) + 32 * (mi & 1) + l32;
                        const int64_t col = n0 + wn * 128 + 32 * ni + 8 * g + 4 * lh;
                        if (hpresent(hh)) store4<OUT>((char*)P.out + (row * P.ldc + col) * OES, v);
                    } else {  // DSTD, transposed C: lane holds 4 consecutive m of column n
                        const int m0 = 32 * mi + 8 * g + 4 * lh;
                        const int64_t n = n0 + wn * 128 + 32 * ni + l32;
                        const int64_t off = n * P.ldc + (int64_t)kBlock * mrow + m0;
                        store4<OUT>((char*)P.out + off * OES, v);
                    }
                }
                // keep the scheduler from hoisting every accumulator read of
                // the epilogue at once (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // slab 0 has been read: slab 3 goes into its buffer while half 0 is
        // flushed
        if constexpr (GLDS && NMI > 2) {
            if (h == 0) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                gslab(3, gbuf);
            }
        }
        // the staged half goes out only when its slot is present (an absent
        // slot's rows belong to the next expert or lie past the bins)
        if constexpr (STAGE && DUAL) {
            const int64_t o =
                ((int64_t)hblk(h) * BR * kBlock + hin(h) * kBlock + wn * 64) * OES;
            if (hpresent(h)) {
                stage_flush_d(region, (char*)P.out + o);
                if constexpr (EPI == kEpiSiluMulSave) {
                    stage_flush_d(region + 8192, (char*)P.aux_out + o);
                    stage_flush_d(region + 16384, (char*)P.aux_out + P.plane * OES + o);
                }
            }
        } else if constexpr (STAGE) {
            if constexpr (EPI == kEpiGeluSave) {
                if (hpresent(h)) {
                    stage_flush(region, (char*)P.aux_out +
                                            ((int64_t)hblk(h) * BR * kBlock + hin(h) * kBlock) * OES,
                                orow);
                    stage_flush(region + 16384, hbase(h), orow);
                }
            } else if constexpr (EPI == kEpiSiluMulBwd) {
                if (hpresent(h)) {
                    stage_flush(region, hbase(h), orow);
                    stage_flush(region + 16384, hbase(h) + P.plane * OES, orow);
                }
            } else if constexpr (EPI == kEpiScatter) {
                // take the rows' assignments and gates (loaded at the start of
                // the epilogue, long landed) before the first store: a wait for
                // them later would also wait for every store issued since
                if (h == 0) {
#pragma unroll
                    for (int hh = 0; hh < NH; ++hh) asm volatile("" ::"v"(sc_a[hh]), "v"(sc_g[hh]));
                }
                if (P.out && hpresent(h)) stage_flush(region, hbase(h), orow);
                scatter_flush(region, h);
            } else {
                if (hpresent(h)) stage_flush(region, hbase(h), orow);
            }
        }
    }
}

struct SplitPlan {
    int full, tail, S;
};

// The SDD's last round, after at least one full round, when at most half the
// CUs would run it: each of its t tiles runs as two half tiles (the row
// tile's first 128 rows, then the rest), 2t workgroups of about two thirds
// of a tile's time each.  The activation needs the whole K sum, so the SDD
// splits along M, not K.
__device__ __forceinline__ SplitPlan sdd_plan(int ntiles, int ncu) {
    SplitPlan p{ntiles, 0, 1};
    if (ncu <= 0 || ntiles < ncu) return p;
    const int tail = ntiles % ncu;
    if (tail == 0 || 2 * tail > ncu) return p;
    return SplitPlan{ntiles - tail, tail, 2};
}

// Split of a DSD launch's last, partly filled round: with ntiles tiles on
// ncu CUs, the tail (ntiles mod ncu tiles) is cut into S K-segments each, S =
// min(ncu / tail, kMaxSplit, units / tail), so the last round runs tail x S
// shares of 1/S of a tile instead of tail whole tiles on a nearly idle chip.
// No split (full = ntiles) when S < 2 or no workspace.  Both launches of a
// split product compute the same plan from the same device-side tile count.
__device__ __forceinline__ SplitPlan split_plan(int ntiles, int ncu, int units) {
    SplitPlan p{ntiles, 0, 1};
    if (ncu <= 0 || units <= 0) return p;
    const int tail = ntiles % ncu;
    if (tail == 0) return p;
    const int S = min(min(ncu / tail, kMaxSplit), units / tail);
    if (S < 2) return p;
    return SplitPlan{ntiles - tail, tail, S};
}

// Whether SDD / DSD tile `tile` (group order) is a half tile: its row
// tile's count of present block rows is at most 128 rows' worth.
template <int MODE, int BR>
__device__ __forceinline__ bool half_tile(const GemmParams& P, int tile, int tn) {
    int tm, tq;
    row_tile_of(P.row_tiles, tile, tn, tm, tq);
    return __builtin_amdgcn_readfirstlane((P.row_tiles[tm] & 3) + 1) <= kBlock / BR;
}

template <int DT, int MODE, bool BK, int EPI, int OUT, bool SWAP, int BR>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmParams P) {
    // the operand ring
    // (GeLU backward, bf16) four 8 KB buffers of the saved derivative
    constexpr bool kGbuf = EPI == kEpiGeluBwd && OUT == kBf16;
    __shared__ __attribute__((aligned(1024))) char
        smem[kLdsBytes + (kGbuf ? 4 * 8192 : 0)];
    if constexpr (MODE == kModeDstd) {
        gemm_tile<DT, MODE, BK, EPI, OUT, SWAP, false, BR>(P, smem, 0, 0, 1, nullptr);
    } else {
        // SDD / DSD: workgroup -> tile, XCD-aware (each XCD a contiguous range
        // of the group order); a split DSD's last round: workgroup -> share
        const int tn = MODE == kModeSdd ? (P.F + 1) / 2 : MODE == kModeSddOne ? P.F : P.ntn;
        const int ntiles = P.meta[3] * tn;
        SplitPlan pl{ntiles, 0, 1};
        if constexpr (MODE == kModeDsd || MODE == kModeDsd2) {
            if (P.ws) pl = split_plan(ntiles, P.ncu, P.ws_units);
        } else if constexpr (MODE == kModeSdd) {
            pl = sdd_plan(ntiles, P.ncu);
        }
        const int b = blockIdx.x;
        int tile, seg = 0, nseg = 1;
        float* part = nullptr;
        if (b < pl.full) {
            tile = xcd_remap(b, pl.full);
        } else if (b < pl.full + pl.tail * pl.S) {
            // the split round: each XCD a contiguous range of (segment, tile)
            // in segment-major order, so the shares it runs at once cover one
            // K-segment of neighbouring tiles and share their operand panels
            const int v = xcd_remap(b - pl.full, pl.tail * pl.S);
            const int i = v % pl.tail;
            seg = v / pl.tail;
            tile = pl.full + i;
            nseg = pl.S;
            if constexpr (MODE == kModeDsd || MODE == kModeDsd2)
                part = P.ws + ((int64_t)i * pl.S + seg) * kSplitFloats;
        } else {
            return;
        }
        if constexpr (MODE == kModeSdd || MODE == kModeDsd || MODE == kModeDsd2) {
            // one call site per body: a half tile, or half `seg` of a split SDD
            // row tile (nothing when the row tile has no second half)
            const bool half = half_tile<MODE, BR>(P, tile, tn);
            bool run_half = half;
            if constexpr (MODE == kModeSdd) {
                if (nseg == 2) {
                    if (seg == 1 && half) return;
                    run_half = true;
                }
            }
            if (run_half) {
                gemm_tile<DT, MODE, BK, EPI, OUT, SWAP, true, BR>(P, smem, tile, seg, nseg, part);
                return;
            }
        }
        gemm_tile<DT, MODE, BK, EPI, OUT, SWAP, false, BR>(P, smem, tile, seg, nseg, part);
    }
}

// The second launch of a split DSD: workgroup i sums the S shares of tail
// tile full + i in segment order (shares as gemm_tile writes them) and
// stores the tile as the plain DSD epilogue does, row-major C.  MODE and BK
// name the product it completes (as gemm_kernel's arguments do) and select
// nothing else.
template <int MODE, bool BK, int OUT, int BR>
__global__ __launch_bounds__(kGemmThreads) void dsd_reduce_kernel(GemmParams P) {
    const SplitPlan pl = split_plan(P.meta[3] * P.ntn, P.ncu, P.ws_units);
    if ((int)blockIdx.x >= pl.tail) return;
    const int tile = pl.full + blockIdx.x;
    int tm, tq;
    row_tile_of(P.row_tiles, tile, P.ntn, tm, tq);
    const int ent = __builtin_amdgcn_readfirstlane(P.row_tiles[tm]);
    const int r0 = ent >> 8, nq = (ent & 3) + 1;
    constexpr int QB = kBlock / BR;
    const bool half = nq <= QB;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1, l32 = lane & 31, lh = lane >> 5;
    const int64_t n0 = (int64_t)tq * 256;
    if (wn == 1 && n0 + 128 >= P.N) return;  // absent N half
    constexpr int OES = OUT == kBf16 ? 2 : 4;
    const float* src = P.ws + (int64_t)blockIdx.x * pl.S * kSplitFloats + wave * (kSplitFloats / 4) +
                       lane * 16;
    const int nmi = half ? 2 : 4;
    for (int mi = 0; mi < nmi; ++mi) {
        // rows of fragment mi inside the tile, and whether its block row is present
        const int hrow = half ? 64 * wm : 128 * wm + 64 * (mi >> 1);
        if (hrow / BR >= nq) continue;
        const int64_t row = (int64_t)BR * r0 + hrow + 32 * (mi & 1) + l32;
        // the 4 x 4 accumulator vectors of row fragment mi, summed share by
        // share (each share's 16 loads in flight together)
        f32x4 v[4][4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[ni][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int sgm = 0; sgm < pl.S; ++sgm) {
            const float* sp = src + (int64_t)sgm * kSplitFloats + mi * 4 * 1024;
            f32x4 x[4][4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) x[ni][q] = *(const f32x4*)(sp + ni * 1024 + 4 * q);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[ni][q][e] += x[ni][q][e];
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t col = n0 + wn * 128 + 32 * ni + 8 * g + 4 * lh;
                const float w[4] = {v[ni][g][0], v[ni][g][1], v[ni][g][2], v[ni][g][3]};
                store4<OUT>((char*)P.out + (row * P.ldc + col) * OES, w);
            }
    }
}

// ----------------------------------------------------------------- launch

template <int DT, int MODE, bool BK, int EPI, int OUT, bool SWAP, int BR>
static hipError_t launch(const GemmParams& p, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<DT, MODE, BK, EPI, OUT, SWAP, BR>), dim3((unsigned)grid),
                       dim3(kGemmThreads), 0, s, p);
    return hipGetLastError();
}

template <int DT, int BR>
static hipError_t dispatch_sdd(const GemmParams& p, int64_t grid, int trans_b, int epi,
                               hipStream_t s) {
    switch (epi) {
    case kEpiNone:
        return trans_b ? launch<DT, kModeSdd, true, kEpiNone, DT, true, BR>(p, grid, s)
                       : launch<DT, kModeSdd, false, kEpiNone, DT, true, BR>(p, grid, s);
    case kEpiGelu:
        if (p.aux_out)
            return trans_b ? launch<DT, kModeSdd, true, kEpiGeluSave, DT, true, BR>(p, grid, s)
                           : launch<DT, kModeSdd, false, kEpiGeluSave, DT, true, BR>(p, grid, s);
        return trans_b ? launch<DT, kModeSdd, true, kEpiGelu, DT, true, BR>(p, grid, s)
                       : launch<DT, kModeSdd, false, kEpiGelu, DT, true, BR>(p, grid, s);
    case kEpiGeluBwd:
        return trans_b ? launch<DT, kModeSdd, true, kEpiGeluBwd, DT, true, BR>(p, grid, s)
                       : launch<DT, kModeSdd, false, kEpiGeluBwd, DT, true, BR>(p, grid, s);
    case kEpiSiluMulBwd:
        return trans_b ? launch<DT, kModeSdd, true, kEpiSiluMulBwd, DT, true, BR>(p, grid, s)
                       : launch<DT, kModeSdd, false, kEpiSiluMulBwd, DT, true, BR>(p, grid, s);
    default:
        return hipErrorInvalidValue;
    }
}

template <int BR>
hipError_t launch_sdd_br(const GemmParams& p, int64_t row_tiles_max, int trans_b, int epi,
                         int dtype, hipStream_t s) {
    if (epi == kEpiSiluMul) {  // dual B: one block per tile, B halves = W1 | W3
        if (trans_b) return hipErrorInvalidValue;
        const int64_t grid = row_tiles_max * p.F;
        if (p.aux_out)
            return dtype == kBf16
                       ? launch<kBf16, kModeSddOne, false, kEpiSiluMulSave, kBf16, true, BR>(p, grid, s)
                       : launch<kF32, kModeSddOne, false, kEpiSiluMulSave, kF32, true, BR>(p, grid, s);
        return dtype == kBf16
                   ? launch<kBf16, kModeSddOne, false, kEpiSiluMul, kBf16, true, BR>(p, grid, s)
                   : launch<kF32, kModeSddOne, false, kEpiSiluMul, kF32, true, BR>(p, grid, s);
    }
    // (+ ncu / 2: the second halves of a split last round)
    const int64_t grid = row_tiles_max * ((p.F + 1) / 2) + p.ncu / 2;
    return dtype == kBf16 ? dispatch_sdd<kBf16, BR>(p, grid, trans_b, epi, s)
                          : dispatch_sdd<kF32, BR>(p, grid, trans_b, epi, s);
}

template <int MODE, int BR>
static hipError_t dispatch_dsd(const GemmParams& p, int64_t grid, int trans_b, int c_dtype,
                               int dtype, hipStream_t s) {
    if (dtype == kF32)
        return trans_b ? launch<kF32, MODE, true, kEpiNone, kF32, true, BR>(p, grid, s)
                       : launch<kF32, MODE, false, kEpiNone, kF32, true, BR>(p, grid, s);
    if (c_dtype == kBf16)
        return trans_b ? launch<kBf16, MODE, true, kEpiNone, kBf16, true, BR>(p, grid, s)
                       : launch<kBf16, MODE, false, kEpiNone, kBf16, true, BR>(p, grid, s);
    return trans_b ? launch<kBf16, MODE, true, kEpiNone, kF32, true, BR>(p, grid, s)
                   : launch<kBf16, MODE, false, kEpiNone, kF32, true, BR>(p, grid, s);
}

template <int MODE, int OUT, int BR>
static void launch_reduce(const GemmParams& p, int trans_b, hipStream_t s) {
    if (trans_b)
        hipLaunchKernelGGL((dsd_reduce_kernel<MODE, true, OUT, BR>), dim3((unsigned)p.ncu),
                           dim3(kGemmThreads), 0, s, p);
    else
        hipLaunchKernelGGL((dsd_reduce_kernel<MODE, false, OUT, BR>), dim3((unsigned)p.ncu),
                           dim3(kGemmThreads), 0, s, p);
}

template <int BR>
hipError_t launch_dsd_br(const GemmParams& p, int64_t row_tiles_max, int trans_b, int c_dtype,
                         int dtype, hipStream_t s) {
    const int64_t grid = row_tiles_max * p.ntn;
    if (p.scat_out) {  // top-1 rows to token order: bf16 throughout, one block set
        if (dtype != kBf16 || c_dtype != kBf16 || p.a2 || p.ws) return hipErrorInvalidValue;
        return trans_b ? launch<kBf16, kModeDsd, true, kEpiScatter, kBf16, true, BR>(p, grid, s)
                       : launch<kBf16, kModeDsd, false, kEpiScatter, kBf16, true, BR>(p, grid, s);
    }
    if (!p.ws)
        return p.a2 ? dispatch_dsd<kModeDsd2, BR>(p, grid, trans_b, c_dtype, dtype, s)
                    : dispatch_dsd<kModeDsd, BR>(p, grid, trans_b, c_dtype, dtype, s);
    // split last round: up to ncu more workgroups for the shares, then the
    // reduction of the split tiles
    if (p.ncu <= 0 || p.ws_units < 2) return hipErrorInvalidValue;
    const int64_t g2 = grid + p.ncu;
    hipError_t e = p.a2 ? dispatch_dsd<kModeDsd2, BR>(p, g2, trans_b, c_dtype, dtype, s)
                        : dispatch_dsd<kModeDsd, BR>(p, g2, trans_b, c_dtype, dtype, s);
    if (e != hipSuccess || grid <= 0) return e;
    const int out = dtype == kF32 ? kF32 : c_dtype;
    if (p.a2) {
        if (out == kBf16) launch_reduce<kModeDsd2, kBf16, BR>(p, trans_b, s);
        else launch_reduce<kModeDsd2, kF32, BR>(p, trans_b, s);
    } else {
        if (out == kBf16) launch_reduce<kModeDsd, kBf16, BR>(p, trans_b, s);
        else launch_reduce<kModeDsd, kF32, BR>(p, trans_b, s);
    }
    return hipGetLastError();
}

template <int BR>
hipError_t launch_dstd_br(const GemmParams& p, int trans_c, int dtype, hipStream_t s) {
    const int64_t grid = (int64_t)p.E * ((p.F + 1) / 2) * p.ntn;
    if (dtype == kF32)
        return trans_c ? launch<kF32, kModeDstd, false, kEpiNone, kF32, false, BR>(p, grid, s)
                       : launch<kF32, kModeDstd, false, kEpiNone, kF32, true, BR>(p, grid, s);
    return trans_c ? launch<kBf16, kModeDstd, false, kEpiNone, kBf16, false, BR>(p, grid, s)
                   : launch<kBf16, kModeDstd, false, kEpiNone, kBf16, true, BR>(p, grid, s);
}

#define BSG_GEMM_INSTANTIATE(BR)                                                              \
    template hipError_t launch_sdd_br<BR>(const GemmParams&, int64_t, int, int, int, hipStream_t); \
    template hipError_t launch_dsd_br<BR>(const GemmParams&, int64_t, int, int, int, hipStream_t); \
    template hipError_t launch_dstd_br<BR>(const GemmParams&, int, int, hipStream_t);

}  // namespace bsg
