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

// The same for two integers at once (one barrier for both).
template <int NW>
__device__ __forceinline__ int2 block_excl_scan2(int2 v, int2* wsum, int2& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int2 inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int ux = __shfl_up(inc.x, off, kWave);
        const int uy = __shfl_up(inc.y, off, kWave);
        if (lane >= off) {
            inc.x += ux;
            inc.y += uy;
        }
    }
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    int2 base = make_int2(0, 0);
    total = make_int2(0, 0);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int2 ws = wsum[w];
        if (w < wave) {
            base.x += ws.x;
            base.y += ws.y;
        }
        total.x += ws.x;
        total.y += ws.y;
    }
    return make_int2(base.x + inc.x - v.x, base.y + inc.y - v.y);
}

}  // namespace bsg
