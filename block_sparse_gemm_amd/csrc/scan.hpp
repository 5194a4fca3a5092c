// Workgroup-wide integer scan shared by the routing and topology kernels.
#pragma once
#include "common.hpp"

namespace bsg {

// Exclusive scan over the NW waves of a workgroup (integers, so exact in any
// order): shuffle scans inside each wave, then one barrier to add the
// earlier waves' totals.  `wsum` is NW ints of LDS; the call holds one
// barrier, so a workgroup calls it at most once between other barriers that
// protect `wsum`.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += u;
    }
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) base += wsum[w];
        total += wsum[w];
    }
    return base + inc - v;
}

}  // namespace bsg
