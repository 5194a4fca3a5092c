#pragma once
// Device code of the topology builder (the hybrid BCSR-COO topology, its
// transpose index and the products' schedules), shared by the topology
// kernel and by the routing kernel that builds the topology in the same
// launch as the placement.  See topology.hip for what is built and why.
#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace bsg {

constexpr int kTopoThreads = 256;

// Largest e in [0, E) with s[e] <= r; s is non-decreasing.  Empty experts
// share their start with the next expert, so this is the owner of r.
__device__ __forceinline__ int owner_of(const int* s, int E, int r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// LDS state of the builder in a workgroup of NT threads: bin starts in
// block rows, first row tile of each expert, and whether a bin is off the
// block grid.
template <int NT>
struct TopoLds {
    int s[kMaxExperts + 1];
    int pp[kMaxExperts + 1];
    int wsum[NT / kWave];
    int misaligned;
};

// s and pp from the bin offsets (in rows, E + 1 values, read from `bins`,
// global memory or LDS); every thread of the NT-thread workgroup takes part
// (barriers inside).
template <int NT>
__device__ __forceinline__ void topo_prepare(const int32_t* bins, int E, int br, TopoLds<NT>& L) {
    const int q = 256 / br;  // block rows per tile
    if (threadIdx.x == 0) L.misaligned = 0;
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += NT) {
        const int b = bins[e];
        L.s[e] = b / br;
        if (b % br) L.misaligned = 1;  // a bin that does not start on the block grid
    }
    __syncthreads();
    // row tiles: expert e's R_e row blocks form ceil(R_e / q) tiles of q
    // consecutive rows (the last one shorter); exclusive scan
    const int per = (E + NT - 1) / NT;
    const int lo = threadIdx.x * per, hi = min(lo + per, E);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += (L.s[e + 1] - L.s[e] + q - 1) / q;
    int total;
    int run = block_excl_scan<NT / kWave>(sum, L.wsum, total);
    for (int e = lo; e < hi; ++e) {
        L.pp[e] = run;
        run += (L.s[e + 1] - L.s[e] + q - 1) / q;
    }
    if (threadIdx.x == NT - 1) L.pp[E] = total;
    __syncthreads();
}

// expert_order: the experts by descending row count (ties: lower id
// first).  One wavefront per expert, wave w of the nw taking part handling
// experts w, w + nw, ...: the expert's place is the number of experts
// ahead of it, counted with one ballot per 64 experts.
template <int NT>
__device__ __forceinline__ void topo_order(const TopoLds<NT>& L, int E, int w, int nw,
                                           int32_t* __restrict__ expert_order) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int g = w; g < E; g += nw) {
        const int rg = L.s[g + 1] - L.s[g];
        int rank = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            bool ahead = false;
            if (e < E) {
                const int re = L.s[e + 1] - L.s[e];
                ahead = re > rg || (re == rg && e < g);
            }
            rank += __popcll(__ballot(ahead));
        }
        if (lane == 0) expert_order[rank] = g;
    }
}

// Entry g of every topology array but expert_order (thread g of the
// launch's grid).
template <int NT>
__device__ __forceinline__ void topo_write(int64_t g, const TopoLds<NT>& L, int E, int F, int br,
                                           int64_t row_blocks_max, int group,
                                           const TopoArrays& o) {
    const int q = 256 / br;
    const int* s = L.s;
    const int* pp = L.pp;
    const int64_t R = s[E];
    const int64_t nnz = R * F;

    if (R > row_blocks_max || L.misaligned) {
        // the routing needs more rows than the topology holds, or its bins
        // are off the block grid: publish an empty topology (every product
        // then writes nothing / zeros) and raise the status flag instead of
        // writing out of bounds
        if (g == 0) {
            o.meta[0] = 0;
            o.meta[1] = 0;
            o.meta[2] = L.misaligned ? 2 : 1;
            o.meta[3] = 0;
        }
        if (g <= row_blocks_max) o.row_ptr[g] = 0;
        if (g <= (int64_t)E * F) o.col_ptr[g] = 0;
        return;
    }
    // from here on R <= row_blocks_max, so every index fits 32 bits (the
    // capacity's nnz_max and E * F are below 2^31) and the divisions below
    // are 32-bit ones
    if (g >= (int64_t)INT32_MAX) return;
    const int gi = (int)g;
    const int Ri = (int)R, nnzi = (int)nnz, EF = E * F;
    if (gi == 0) {
        o.meta[0] = nnzi;
        o.meta[1] = Ri;
        o.meta[2] = 0;
        o.meta[3] = pp[E];
    }
    if (gi < pp[E]) {
        // the expert's tiles go in groups of `group` (the last one shorter):
        // the products take a group's tiles together
        const int e = owner_of(pp, E, gi);
        const int j = gi - pp[e];
        const int Re = s[e + 1] - s[e];
        const int r0 = s[e] + q * j;
        const int ntiles = pp[e + 1] - pp[e];
        const int off = j % group;
        const int size = min(group, ntiles - (j - off));
        const int rows = min(q, Re - q * j);
        o.row_tiles[gi] = (r0 << 8) | ((size - 1) << 5) | (off << 2) | (rows - 1);
    }
    // BCSR block pointer: every non-empty row block holds F blocks
    if (g <= row_blocks_max) o.row_ptr[gi] = min(gi, Ri) * F;
    if (gi < nnzi) {
        // BCSR entry g = (row block r, j-th block of the row) + its COO row
        const int r = (int)((unsigned)gi / (unsigned)F);
        const int j = gi - r * F;
        const int e = owner_of(s, E, r);
        o.col_idx[gi] = e * F + j;
        o.row_idx[gi] = r;
        // transpose entry g: expert e' owns positions [s_e' F, s_(e'+1) F),
        // so e' is the owner of row block g / F, the same e; inside its
        // range, column j' holds R_e' blocks in ascending row order
        const int Re = s[e + 1] - s[e];
        const int local = gi - s[e] * F;
        const int jt = (int)((unsigned)local / (unsigned)Re);
        const int it = local - jt * Re;
        o.trans_idx[gi] = (s[e] + it) * F + jt;
    }
    if (gi < EF) {
        const int e = (int)((unsigned)gi / (unsigned)F);
        const int j = gi - e * F;
        o.col_ptr[gi] = s[e] * F + j * (s[e + 1] - s[e]);
    }
    if (gi == EF) o.col_ptr[gi] = nnzi;
}

// Threads a topology of this capacity needs: one per entry of its longest
// array.
inline int64_t topo_threads(int E, int F, int64_t row_blocks_max, int64_t row_tiles_max) {
    int64_t n = row_blocks_max * F;
    if (row_tiles_max > n) n = row_tiles_max;
    if (row_blocks_max + 1 > n) n = row_blocks_max + 1;
    if ((int64_t)E * F + 1 > n) n = (int64_t)E * F + 1;
    if (E > n) n = E;
    return n;
}

}  // namespace bsg
