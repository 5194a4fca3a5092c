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
// finds the owner of a row block by binary search; an expert's place in
// the descending order is counted by one wavefront with ballots.  The same
// device code (topology.hpp) also runs inside the routing's placement
// launch, which forms the bins itself.
#include "topology.hpp"

namespace bsg {

__global__ __launch_bounds__(kTopoThreads) void build_topology_kernel(
    const int32_t* __restrict__ bin_offsets, int E, int F, int br, int64_t row_blocks_max,
    int group, TopoArrays o) {
    __shared__ TopoLds<kTopoThreads> L;
    topo_prepare(bin_offsets, E, br, L);
    topo_order(L, E, (int)(blockIdx.x * (kTopoThreads / kWave) + threadIdx.x / kWave),
               (int)(gridDim.x * (kTopoThreads / kWave)), o.expert_order);
    topo_write((int64_t)blockIdx.x * kTopoThreads + threadIdx.x, L, E, F, br, row_blocks_max,
               group, o);
}

hipError_t launch_build_topology(const int32_t* bin_offsets, int E, int F, int br,
                                 int64_t row_blocks_max, int64_t row_tiles_max, int32_t* row_ptr,
                                 int32_t* col_idx, int32_t* row_idx, int32_t* col_ptr,
                                 int32_t* trans_idx, int32_t* row_tiles, int32_t* expert_order,
                                 int32_t* meta, int group, hipStream_t stream) {
    const int64_t n = topo_threads(E, F, row_blocks_max, row_tiles_max);
    const int grid = (int)((n + kTopoThreads - 1) / kTopoThreads);
    const TopoArrays o{row_ptr, col_idx, row_idx, col_ptr, trans_idx, row_tiles, expert_order, meta};
    hipLaunchKernelGGL(build_topology_kernel, dim3(grid), dim3(kTopoThreads), 0, stream,
                       bin_offsets, E, F, br, row_blocks_max, group, o);
    return hipGetLastError();
}

}  // namespace bsg
