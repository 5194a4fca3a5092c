// Topology + transpose metadata in one launch.
//
// George Lin's Blog (MegaBlocks/FlexMoE post): section 1.3 defines the
// hybrid BCSR-COO format (BCSR row pointer + column index, plus a
// materialised row index per nonzero block) and the transpose index (the
// same blocks listed in column order, no data copied); section 1.4 builds
// this metadata, mapping each (expert, token-row range) to its nonzero
// blocks, together with the transpose metadata in a single kernel.
//
// It also emits the schedules the products run on: the row tiles (the
// consecutive block rows of one expert share their column list, so a
// 256-row tile of two 128-row or four 64-row block rows reads one set of
// weight columns), and the experts in descending order of their row count,
// so the weight-gradient product, whose tile cost grows with the expert's
// rows, starts its longest tiles first.
//
// The first layer's output is block-diagonal: row block r (br rows: 128,
// or 64 for the block-size study's bins of 64 rows) belongs to the expert
// whose bin holds row br * r, and that expert owns the F column blocks
// e*F .. e*F + F - 1.  So every entry is computed independently from the
// bin offsets: thread g fills row_ptr[g], BCSR entry g and transpose entry
// g.  Each workgroup first stages s_e = bin_offsets[e] / br in LDS and
// finds the owner of a row block by binary search.
#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace bsg {

constexpr int kTopoThreads = 256;

// Largest e in [0, E) with s[e] <= r; s is non-decreasing.  Empty experts
// share their start with the next expert, so this is the owner of r.
__device__ __forceinline__ int owner_of(const int* s, int E, int64_t r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kTopoThreads) void build_topology_kernel(
    const int32_t* __restrict__ bin_offsets, int E, int F, int br, int64_t row_blocks_max,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int32_t* __restrict__ row_idx,
    int32_t* __restrict__ col_ptr, int32_t* __restrict__ trans_idx,
    int32_t* __restrict__ row_tiles, int32_t* __restrict__ expert_order,
    int32_t* __restrict__ meta, int group) {
    __shared__ int s[kMaxExperts + 1];   // bin start in row blocks
    __shared__ int pp[kMaxExperts + 1];  // first row tile of each expert
    __shared__ int wsum[kTopoThreads / kWave];
    __shared__ int misaligned;
    const int q = 256 / br;  // block rows per tile
    if (threadIdx.x == 0) misaligned = 0;
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += kTopoThreads) {
        const int b = bin_offsets[e];
        s[e] = b / br;
        if (b % br) misaligned = 1;  // a bin that does not start on the block grid
    }
    __syncthreads();
    // row tiles: expert e's R_e row blocks form ceil(R_e / q) tiles of q
    // consecutive rows (the last one shorter); exclusive scan
    const int per = (E + kTopoThreads - 1) / kTopoThreads;
    const int lo = threadIdx.x * per, hi = min(lo + per, E);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += (s[e + 1] - s[e] + q - 1) / q;
    int total;
    int run = block_excl_scan<kTopoThreads / kWave>(sum, wsum, total);
    for (int e = lo; e < hi; ++e) {
        pp[e] = run;
        run += (s[e + 1] - s[e] + q - 1) / q;
    }
    if (threadIdx.x == kTopoThreads - 1) pp[E] = total;
    __syncthreads();
    const int64_t R = s[E];
    const int64_t nnz = R * F;
    const int64_t g = (int64_t)blockIdx.x * kTopoThreads + threadIdx.x;

    // expert g's place in descending row count (ties: lower id first)
    if (g < E) {
        const int rg = s[g + 1] - s[g];
        int rank = 0;
        for (int e = 0; e < E; ++e) {
            const int re = s[e + 1] - s[e];
            rank += (re > rg || (re == rg && e < g)) ? 1 : 0;
        }
        expert_order[rank] = (int32_t)g;
    }

    if (R > row_blocks_max || misaligned) {
        // the routing needs more rows than the topology holds, or its bins
        // are off the block grid: publish an empty topology (every product
        // then writes nothing / zeros) and raise the status flag instead of
        // writing out of bounds
        if (g == 0) {
            meta[0] = 0;
            meta[1] = 0;
            meta[2] = misaligned ? 2 : 1;
            meta[3] = 0;
        }
        if (g <= row_blocks_max) row_ptr[g] = 0;
        if (g <= (int64_t)E * F) col_ptr[g] = 0;
        return;
    }
    if (g == 0) {
        meta[0] = (int32_t)nnz;
        meta[1] = (int32_t)R;
        meta[2] = 0;
        meta[3] = pp[E];
    }
    if (g < pp[E]) {
        // the expert's tiles go in groups of `group` (the last one shorter):
        // the products take a group's tiles together
        const int e = owner_of(pp, E, g);
        const int j = (int)(g - pp[e]);
        const int Re = s[e + 1] - s[e];
        const int r0 = s[e] + q * j;
        const int ntiles = pp[e + 1] - pp[e];
        const int off = j % group;
        const int size = min(group, ntiles - (j - off));
        const int rows = min(q, Re - q * j);
        row_tiles[g] = (r0 << 8) | ((size - 1) << 5) | (off << 2) | (rows - 1);
    }
    // BCSR block pointer: every non-empty row block holds F blocks
    if (g <= row_blocks_max) row_ptr[g] = (int32_t)((g < R ? g : R) * F);
    if (g < nnz) {
        // BCSR entry g = (row block r, j-th block of the row) + its COO row
        const int64_t r = g / F;
        const int j = (int)(g % F);
        const int e = owner_of(s, E, r);
        col_idx[g] = e * F + j;
        row_idx[g] = (int32_t)r;
        // transpose entry g: expert e' owns positions [s_e' F, s_(e'+1) F);
        // inside it, column j' holds R_e' blocks in ascending row order
        const int et = owner_of(s, E, g / F);
        const int64_t Re = s[et + 1] - s[et];
        const int64_t local = g - (int64_t)s[et] * F;
        const int64_t jt = local / Re, it = local % Re;
        trans_idx[g] = (int32_t)((s[et] + it) * F + jt);
    }
    if (g < (int64_t)E * F) {
        const int e = (int)(g / F);
        const int j = (int)(g % F);
        col_ptr[g] = (int32_t)((int64_t)s[e] * F + (int64_t)j * (s[e + 1] - s[e]));
    }
    if (g == (int64_t)E * F) col_ptr[g] = (int32_t)nnz;
}

hipError_t launch_build_topology(const int32_t* bin_offsets, int E, int F, int br,
                                 int64_t row_blocks_max, int64_t row_tiles_max, int32_t* row_ptr,
                                 int32_t* col_idx, int32_t* row_idx, int32_t* col_ptr,
                                 int32_t* trans_idx, int32_t* row_tiles, int32_t* expert_order,
                                 int32_t* meta, int group, hipStream_t stream) {
    int64_t n = row_blocks_max * F;
    if (row_tiles_max > n) n = row_tiles_max;
    if (row_blocks_max + 1 > n) n = row_blocks_max + 1;
    if ((int64_t)E * F + 1 > n) n = (int64_t)E * F + 1;
    if (E > n) n = E;
    const int grid = (int)((n + kTopoThreads - 1) / kTopoThreads);
    hipLaunchKernelGGL(build_topology_kernel, dim3(grid), dim3(kTopoThreads), 0, stream,
                       bin_offsets, E, F, br, row_blocks_max, row_ptr, col_idx, row_idx, col_ptr,
                       trans_idx, row_tiles, expert_order, meta, group);
    return hipGetLastError();
}

}  // namespace bsg
