// Block-sparse products on CDNA4 matrix cores: SDD, DSD and DSTD.
//
// George Lin's Blog (MegaBlocks/FlexMoE post):
//  - section 1.2: one block-sparse product replaces the per-expert batched
//    GEMMs; the first layer is SDD (a dense x dense product sampled at the
//    nonzero blocks), then the activation, then DSD (sparse x dense);
//  - section 1.3: 128 x 128 blocks; BCSR walks a block row in order (DSD),
//    the materialised row index gives random access to any block (SDD),
//    and the transpose index lists each column's blocks for DSTD, the
//    weight gradient (sparse^T x dense).
//
// One kernel template serves all three.  A workgroup (256 threads = 4
// wave64s) computes a 128 x 256 output tile with v_mfma_f32_32x32x16_bf16
// (fp32 operands: v_mfma_f32_32x32x2_f32), fp32 accumulation:
//   SDD   two consecutive nonzero blocks of one block row (random access
//         through row_idx), K = d, B columns from col_idx;
//   DSD   one block row x 256 output columns, K walks the row's blocks via
//         row_ptr / col_idx;
//   DSTD  one block column x 256 output columns, K walks the column's
//         blocks via col_ptr / trans_idx, their rows via row_idx.
// Operands are staged through LDS in 128-byte rows (64 bf16 or 32 fp32 of
// K per row), K-contiguous, with an XOR swizzle of the 16-byte chunks so
// that both the 16-byte fragment reads and the stores are bank-conflict
// free.  Operands whose contiguous dimension is M or N are transposed in
// registers (8 x 8 bf16 / 4 x 4 fp32) on their way into LDS.  Global loads
// for K-tile i+1 are in flight while the matrix cores work on K-tile i.
//
// The MFMA operands are swapped (B fragment first) when the output is
// row-major: each lane then holds 4 consecutive columns of one output row
// and writes them with one 8- or 16-byte store.
//
// Workgroup ids are remapped so each of the 8 XCDs runs a contiguous range
// of tiles: consecutive tiles share the A panel (SDD, DSD) or the block
// column (DSTD), which then stays in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace bsg {

constexpr int kGemmThreads = 256;
constexpr int kTileM = 128;
constexpr int kTileN = 256;
constexpr int kChunks = 8;  // 16-byte chunks per 128-byte LDS row
constexpr int kLdsRows = kTileM + kTileN;

template <int DT>
struct Elt;
template <>
struct Elt<kBf16> {
    static constexpr int kVec = 8;   // elements per 16 bytes
    static constexpr int kKt = 64;   // K per LDS row
    static constexpr int kBytes = 2;
};
template <>
struct Elt<kF32> {
    static constexpr int kVec = 4;
    static constexpr int kKt = 32;
    static constexpr int kBytes = 4;
};

__device__ __forceinline__ int lds_idx(int row, int q) {
    return row * kChunks + (q ^ ((row ^ (row >> 3)) & 7));
}

// ------------------------------------------------------------ LDS loaders

// NP panels of 128 rows, K contiguous (row stride ld bytes); 4 chunks per
// thread per panel.
template <int NP>
struct KLoader {
    u32x4 r[4 * NP];
    __device__ __forceinline__ void load(const char* b0, const char* b1, int64_t ld0, int64_t ld1,
                                         bool p0, bool p1) {
        const int q = threadIdx.x & 7, row = threadIdx.x >> 3;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const char* b = p ? b1 : b0;
            const int64_t ld = p ? ld1 : ld0;
            if (p ? p1 : p0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    r[4 * p + i] = *(const u32x4*)(b + (int64_t)(row + 32 * i) * ld + q * 16);
            }
        }
    }
    __device__ __forceinline__ void store(u32x4* lds, int row0, bool p0, bool p1) const {
        const int q = threadIdx.x & 7, row = threadIdx.x >> 3;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (p ? p1 : p0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds[lds_idx(row0 + 128 * p + row + 32 * i, q)] = r[4 * p + i];
            }
        }
    }
};

// NP panels of KT k-rows x 128 M/N columns, M/N contiguous (k stride ld
// bytes).  A thread moves V k-rows x V columns (V = elements per 16 bytes)
// and transposes them in registers; when there are fewer such blocks than
// threads, two threads share a block, each taking V/2 of its k-rows.
template <int DT, int NP>
struct MNLoader {
    static constexpr int V = Elt<DT>::kVec;
    static constexpr int MO = 128 / V;
    static constexpr int BPP = (Elt<DT>::kKt / V) * MO;  // blocks per panel
    static constexpr int NB = NP * BPP;
    static constexpr int SPLIT = NB >= kGemmThreads ? 1 : kGemmThreads / NB;
    static constexpr int RV = V / SPLIT;                 // k-rows per thread and block
    static constexpr int NBT = (NB * SPLIT + kGemmThreads - 1) / kGemmThreads;
    u32x4 r[NBT][RV];

    __device__ __forceinline__ void coords(int s, int& blk, int& sh) const {
        const int t = threadIdx.x + kGemmThreads * s;
        blk = t % NB;
        sh = t / NB;  // which V/SPLIT k-rows of the block (0 when SPLIT == 1)
    }

    __device__ __forceinline__ void load(const char* b0, const char* b1, int64_t ld0, int64_t ld1,
                                         bool p0, bool p1) {
#pragma unroll
        for (int s = 0; s < NBT; ++s) {
            int blk, sh;
            coords(s, blk, sh);
            const int p = blk / BPP;
            const int rem = blk % BPP, ko = rem / MO, mo = rem % MO;
            if (p ? p1 : p0) {
                const char* b = p ? b1 : b0;
                const int64_t ld = p ? ld1 : ld0;
#pragma unroll
                for (int v = 0; v < RV; ++v)
                    r[s][v] = *(const u32x4*)(b + (int64_t)(ko * V + sh * RV + v) * ld + mo * 16);
            }
        }
    }

    __device__ __forceinline__ void store(u32x4* lds, int row0, bool p0, bool p1) const {
#pragma unroll
        for (int s = 0; s < NBT; ++s) {
            int blk, sh;
            coords(s, blk, sh);
            const int p = blk / BPP;
            const int rem = blk % BPP, ko = rem / MO, mo = rem % MO;
            if (p ? p1 : p0) {
#pragma unroll
                for (int m = 0; m < V; ++m) {
                    u32x4* dst = &lds[lds_idx(row0 + 128 * p + mo * V + m, ko)];
                    if constexpr (DT == kBf16) {
                        // dword i of column m = (k = 2i, k = 2i + 1) of this thread's rows
                        uint32_t w[RV / 2];
#pragma unroll
                        for (int i = 0; i < RV / 2; ++i) {
                            const uint32_t lo = r[s][2 * i][m >> 1], hi = r[s][2 * i + 1][m >> 1];
                            w[i] = (m & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                           : ((lo & 0xffffu) | (hi << 16));
                        }
                        if constexpr (RV == 8)
                            *dst = u32x4{w[0], w[1], w[2], w[3]};
                        else
                            ((u32x2*)dst)[sh] = u32x2{w[0], w[1]};
                    } else {
                        static_assert(SPLIT == 1, "fp32 blocks are never split");
                        *dst = u32x4{r[s][0][m], r[s][1][m], r[s][2][m], r[s][3][m]};
                    }
                }
            }
        }
    }
};

template <int DT, bool KC, int NP>
struct LoaderSel {
    using type = KLoader<NP>;
};
template <int DT, int NP>
struct LoaderSel<DT, false, NP> {
    using type = MNLoader<DT, NP>;
};

// --------------------------------------------------------------- MFMA step

template <int DT>
__device__ __forceinline__ void mma(f32x16& acc, u32x4 x, u32x4 y);

template <>
__device__ __forceinline__ void mma<kBf16>(f32x16& acc, u32x4 x, u32x4 y) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                  __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
}

// fp32: a 16-byte chunk holds 4 K values; lane half h of chunk pair c uses
// k = 8c + 4h + s in step s, for both operands alike.
template <>
__device__ __forceinline__ void mma<kF32>(f32x16& acc, u32x4 x, u32x4 y) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(x[s]), __uint_as_float(y[s]),
                                                   acc, 0, 0, 0);
}

// ------------------------------------------------------------- epilogues

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

// ----------------------------------------------------------------- kernel

// Block and source row of K-block p (DSD: block of the row and its column;
// DSTD: block of the column and its row), fetched ahead of use so the index
// latency hides behind the MFMA work.
struct BlockIdx {
    int blk, row;
};

// MODE: kModeSdd (pairs of blocks of one row; F even so a pair never
// straddles two rows), kModeSddOne (one block per tile, also the dual-B
// SwiGLU form), kModeDsd, kModeDstd.
template <int DT, int MODE, bool BK, int EPI, int OUT, bool SWAP>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(GemmParams P) {
    constexpr int ES = Elt<DT>::kBytes;
    constexpr int KT = Elt<DT>::kKt;
    constexpr int KPB = kBlock / KT;  // K-tiles per block
    constexpr int OES = OUT == kBf16 ? 2 : 4;
    constexpr bool AK = MODE != kModeDstd;  // A operand K-contiguous?
    constexpr bool DUAL = EPI == kEpiSiluMul;
    constexpr bool SDD = MODE == kModeSdd || MODE == kModeSddOne;
    using ALoad = typename LoaderSel<DT, AK, 1>::type;
    using BLoad = typename LoaderSel<DT, BK, 2>::type;

    __shared__ u32x4 lds[kLdsRows * kChunks];

    // ---- tile count (device-side sizes) and XCD-aware remap
    const int nnz = P.meta[0];
    int ntiles;
    if constexpr (MODE == kModeSdd) ntiles = nnz / 2;
    else if constexpr (MODE == kModeSddOne) ntiles = nnz;
    else if constexpr (MODE == kModeDsd) ntiles = P.meta[1] * P.ntn;
    else ntiles = P.ncols * P.ntn;
    if ((int)blockIdx.x >= ntiles) return;
    const int tile = xcd_remap(blockIdx.x, ntiles);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lh = lane >> 5;

    // ---- tile -> output rows / blocks
    int row;          // SDD, DSD: block row; DSTD: block column
    int blk0 = 0, blk1 = 0;
    bool bp1;         // second 128-wide half of B / of the output present
    int nt = 0;
    if constexpr (MODE == kModeSdd) {
        blk0 = 2 * tile;
        blk1 = blk0 + 1;
        row = P.row_idx[blk0];  // COO row index: random access to any block
        bp1 = true;
    } else if constexpr (MODE == kModeSddOne) {
        blk0 = blk1 = tile;
        row = P.row_idx[tile];
        bp1 = DUAL;
    } else {
        row = tile / P.ntn;
        nt = tile % P.ntn;
        bp1 = nt * kTileN + 128 < P.N;
    }
    int bcol0 = 0, bcol1 = 0;
    if constexpr (SDD) {
        bcol0 = P.col_idx[blk0];
        bcol1 = DUAL ? bcol0 : (bp1 ? P.col_idx[blk1] : 0);
    }
    // K extent
    int nk, kbase = 0;
    if constexpr (SDD) {
        nk = P.K / KT;
    } else if constexpr (MODE == kModeDsd) {
        kbase = P.row_ptr[row];
        nk = (P.row_ptr[row + 1] - kbase) * KPB;
    } else {
        kbase = P.col_ptr[row];
        nk = (P.col_ptr[row + 1] - kbase) * KPB;
    }
    const int nblk = nk / KPB;

    auto fetch_blk = [&](int p) -> int {
        if constexpr (MODE == kModeDsd) return kbase + p;
        else return P.trans_idx[kbase + p];
    };
    auto fetch_row = [&](int b) -> int {
        if constexpr (MODE == kModeDsd) return P.col_idx[b];
        else return P.row_idx[b];
    };
    BlockIdx cur{0, 0}, nx1{0, 0};
    int nx2blk = 0;
    if constexpr (!SDD) {
        if (nblk > 0) {
            cur.blk = fetch_blk(0);
            cur.row = fetch_row(cur.blk);
        }
        if (nblk > 1) {
            nx1.blk = fetch_blk(1);
            nx1.row = fetch_row(nx1.blk);
        }
        if (nblk > 2) nx2blk = fetch_blk(2);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    ALoad la;
    BLoad lb;
    // issue the global loads of K-tile kt (block indices in `cur`)
    auto issue = [&](int kt) {
        const int koff = (kt % KPB) * KT;
        if constexpr (SDD) {
            const char* a = (const char*)P.a + ((int64_t)kBlock * row * P.lda + (int64_t)kt * KT) * ES;
            la.load(a, a, P.lda * ES, 0, true, false);
            const char* bs0 = (const char*)P.b;
            const char* bs1 = DUAL ? (const char*)P.b2 : (const char*)P.b;
            if constexpr (BK) {
                const char* p0 = bs0 + ((int64_t)kBlock * bcol0 * P.ldb + (int64_t)kt * KT) * ES;
                const char* p1 = bs1 + ((int64_t)kBlock * bcol1 * P.ldb + (int64_t)kt * KT) * ES;
                lb.load(p0, p1, P.ldb * ES, P.ldb * ES, true, bp1);
            } else {
                const char* p0 = bs0 + ((int64_t)kt * KT * P.ldb + (int64_t)kBlock * bcol0) * ES;
                const char* p1 = bs1 + ((int64_t)kt * KT * P.ldb + (int64_t)kBlock * bcol1) * ES;
                lb.load(p0, p1, P.ldb * ES, P.ldb * ES, true, bp1);
            }
        } else if constexpr (MODE == kModeDsd) {
            const char* a = (const char*)P.a + ((int64_t)cur.blk * kBlock * kBlock + koff) * ES;
            la.load(a, a, kBlock * ES, 0, true, false);
            const int64_t krow = (int64_t)kBlock * cur.row + koff;
            const int64_t n0 = (int64_t)nt * kTileN;
            if constexpr (BK) {
                const char* p0 = (const char*)P.b + (n0 * P.ldb + krow) * ES;
                lb.load(p0, p0 + 128 * P.ldb * ES, P.ldb * ES, P.ldb * ES, true, bp1);
            } else {
                const char* p0 = (const char*)P.b + (krow * P.ldb + n0) * ES;
                lb.load(p0, p0 + 128 * ES, P.ldb * ES, P.ldb * ES, true, bp1);
            }
        } else {  // DSTD: A = block^T (M contiguous), B = dmat rows (N contiguous)
            const char* a = (const char*)P.a +
                            ((int64_t)cur.blk * kBlock * kBlock + (int64_t)koff * kBlock) * ES;
            la.load(a, a, kBlock * ES, 0, true, false);
            const int64_t drow = (int64_t)kBlock * cur.row + koff;
            const char* p0 = (const char*)P.b + (drow * P.ldb + (int64_t)nt * kTileN) * ES;
            lb.load(p0, p0 + 128 * ES, P.ldb * ES, P.ldb * ES, true, bp1);
        }
    };
    // before issuing K-tile kt_next: rotate the prefetched block indices
    auto advance = [&](int kt_next) {
        if constexpr (!SDD) {
            if (kt_next % KPB == 0) {
                const int p = kt_next / KPB;
                cur = nx1;
                nx1.blk = nx2blk;
                if (p + 1 < nblk) nx1.row = fetch_row(nx1.blk);
                if (p + 2 < nblk) nx2blk = fetch_blk(p + 2);
            }
        }
    };

    const bool active = wn == 0 || bp1;
    int brow[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        if constexpr (DUAL)  // gate columns in sub-tiles 0,1, up columns in 2,3
            brow[ni] = kTileM + (ni < 2 ? wn * 64 + 32 * ni : 128 + wn * 64 + 32 * (ni - 2));
        else
            brow[ni] = kTileM + wn * 128 + 32 * ni;
    }

    if (nk > 0) issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();  // every wave is done reading the previous K-tile
        la.store(lds, 0, true, false);
        lb.store(lds, kTileM, true, bp1);
        __syncthreads();
        if (kt + 1 < nk) {
            advance(kt + 1);
            issue(kt + 1);
        }
        if (active) {
#pragma unroll
            for (int c = 0; c < kChunks / 2; ++c) {
                const int q = 2 * c + lh;
                u32x4 af[2], bf[4];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) af[mi] = lds[lds_idx(wm * 64 + 32 * mi + l32, q)];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bf[ni] = lds[lds_idx(brow[ni] + l32, q)];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        if constexpr (SWAP) mma<DT>(acc[mi][ni], bf[ni], af[mi]);
                        else mma<DT>(acc[mi][ni], af[mi], bf[ni]);
                    }
            }
        }
    }
    if (!active) return;

    // ---- epilogue
    const int oblk = (MODE == kModeSdd && wn == 1) ? blk1 : blk0;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int mrow = wm * 64 + 32 * mi;  // first row of the 32 x 32 sub-tile
#pragma unroll
        for (int ni = 0; ni < (DUAL ? 2 : 4); ++ni) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) v[s] = acc[mi][ni][4 * g + s];
                if constexpr (SDD) {
                    // block-major output: (m, n) of block b at b*16384 + m*128 + n
                    const int m = mrow + l32;
                    int nloc;
                    if constexpr (DUAL) {
                        nloc = wn * 64 + 32 * ni + 8 * g + 4 * lh;
#pragma unroll
                        for (int s = 0; s < 4; ++s) v[s] = silu_f(v[s]) * acc[mi][ni + 2][4 * g + s];
                    } else {
                        nloc = 32 * ni + 8 * g + 4 * lh;
                    }
                    const int64_t off = (int64_t)oblk * kBlock * kBlock + m * kBlock + nloc;
                    if constexpr (EPI == kEpiGelu) {
                        if (P.aux_out) store4<OUT>((char*)P.aux_out + off * OES, v);
#pragma unroll
                        for (int s = 0; s < 4; ++s) v[s] = gelu_f(v[s]);
                    } else if constexpr (EPI == kEpiGeluBwd) {
                        float h[4];
                        load4<OUT>((const char*)P.aux_in + off * OES, h);
#pragma unroll
                        for (int s = 0; s < 4; ++s) v[s] *= gelu_grad_f(h[s]);
                    }
                    store4<OUT>((char*)P.out + off * OES, v);
                } else if constexpr (SWAP) {  // DSD, or DSTD with row-major C
                    const int m = mrow + l32;
                    const int64_t col = (int64_t)nt * kTileN + wn * 128 + 32 * ni + 8 * g + 4 * lh;
                    const int64_t off = ((int64_t)kBlock * row + m) * P.ldc + col;
                    store4<OUT>((char*)P.out + off * OES, v);
                } else {  // DSTD, transposed C: lane holds 4 consecutive m of column n
                    const int m0 = mrow + 8 * g + 4 * lh;
                    const int64_t n = (int64_t)nt * kTileN + wn * 128 + 32 * ni + l32;
                    const int64_t off = n * P.ldc + (int64_t)kBlock * row + m0;
                    store4<OUT>((char*)P.out + off * OES, v);
                }
            }
        }
    }
}

// ----------------------------------------------------------------- launch

template <int DT, int MODE, bool BK, int EPI, int OUT, bool SWAP>
static hipError_t launch(const GemmParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<DT, MODE, BK, EPI, OUT, SWAP>), dim3(grid), dim3(kGemmThreads),
                       0, s, p);
    return hipGetLastError();
}

template <int DT, int MODE>
static hipError_t dispatch_sdd(const GemmParams& p, int grid, int trans_b, int epi, hipStream_t s) {
    switch (epi) {
    case kEpiNone:
        return trans_b ? launch<DT, MODE, true, kEpiNone, DT, true>(p, grid, s)
                       : launch<DT, MODE, false, kEpiNone, DT, true>(p, grid, s);
    case kEpiGelu:
        return trans_b ? launch<DT, MODE, true, kEpiGelu, DT, true>(p, grid, s)
                       : launch<DT, MODE, false, kEpiGelu, DT, true>(p, grid, s);
    case kEpiGeluBwd:
        return trans_b ? launch<DT, MODE, true, kEpiGeluBwd, DT, true>(p, grid, s)
                       : launch<DT, MODE, false, kEpiGeluBwd, DT, true>(p, grid, s);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_sdd(const GemmParams& p, int64_t nnz_max, int F, int trans_b, int epi,
                      int dtype, hipStream_t s) {
    if (epi == kEpiSiluMul) {  // dual B: one block per tile, both halves = gate | up
        if (trans_b || nnz_max <= 0) return trans_b ? hipErrorInvalidValue : hipSuccess;
        return dtype == kBf16
                   ? launch<kBf16, kModeSddOne, false, kEpiSiluMul, kBf16, true>(p, (int)nnz_max, s)
                   : launch<kF32, kModeSddOne, false, kEpiSiluMul, kF32, true>(p, (int)nnz_max, s);
    }
    if (F % 2 == 0) {  // every row holds F blocks: consecutive pairs stay in one row
        const int grid = (int)(nnz_max / 2);
        if (grid <= 0) return hipSuccess;
        return dtype == kBf16 ? dispatch_sdd<kBf16, kModeSdd>(p, grid, trans_b, epi, s)
                              : dispatch_sdd<kF32, kModeSdd>(p, grid, trans_b, epi, s);
    }
    const int grid = (int)nnz_max;
    if (grid <= 0) return hipSuccess;
    return dtype == kBf16 ? dispatch_sdd<kBf16, kModeSddOne>(p, grid, trans_b, epi, s)
                          : dispatch_sdd<kF32, kModeSddOne>(p, grid, trans_b, epi, s);
}

hipError_t launch_dsd(const GemmParams& p, int64_t row_blocks_max, int trans_b, int c_dtype,
                      int dtype, hipStream_t s) {
    const int64_t grid = row_blocks_max * p.ntn;
    if (grid <= 0) return hipSuccess;
    if (dtype == kF32) {
        return trans_b ? launch<kF32, kModeDsd, true, kEpiNone, kF32, true>(p, (int)grid, s)
                       : launch<kF32, kModeDsd, false, kEpiNone, kF32, true>(p, (int)grid, s);
    }
    if (c_dtype == kBf16)
        return trans_b ? launch<kBf16, kModeDsd, true, kEpiNone, kBf16, true>(p, (int)grid, s)
                       : launch<kBf16, kModeDsd, false, kEpiNone, kBf16, true>(p, (int)grid, s);
    return trans_b ? launch<kBf16, kModeDsd, true, kEpiNone, kF32, true>(p, (int)grid, s)
                   : launch<kBf16, kModeDsd, false, kEpiNone, kF32, true>(p, (int)grid, s);
}

hipError_t launch_dstd(const GemmParams& p, int trans_c, int dtype, hipStream_t s) {
    const int64_t grid = (int64_t)p.ncols * p.ntn;
    if (grid <= 0) return hipSuccess;
    if (dtype == kF32)
        return trans_c ? launch<kF32, kModeDstd, false, kEpiNone, kF32, false>(p, (int)grid, s)
                       : launch<kF32, kModeDstd, false, kEpiNone, kF32, true>(p, (int)grid, s);
    return trans_c ? launch<kBf16, kModeDstd, false, kEpiNone, kBf16, false>(p, (int)grid, s)
                   : launch<kBf16, kModeDstd, false, kEpiNone, kBf16, true>(p, (int)grid, s);
}

}  // namespace bsg
