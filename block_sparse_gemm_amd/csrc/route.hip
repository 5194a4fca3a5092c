// Routing: gate + router, histogram, padded bins and stable placement.
//
// George Lin's Blog (MegaBlocks/FlexMoE post), section 1.4: tokens are
// routed to experts and regrouped from batch order into expert order, each
// group padded to a multiple of the 128 block size (section 1.3), or of a
// coarser bin (256 rows) for the block-size study.  The
// pages leave the gate's form open; this follows top-k on the logits with a
// softmax gate.
//
// Three launches, no atomics on global memory, so every integer result is
// identical on every run:
//   1. route_topk     one workgroup per 64-token chunk, one wavefront per
//                     token at a time (4 each, loaded up front): top-k by
//                     wave reductions, softmax gate; an LDS histogram.  Up
//                     to 64 experts and top-16 (route_topk_seg): the 4
//                     tokens of a wave side by side, 16 lanes each.
//   2. route_scan     one workgroup per expert: exclusive scan of that
//                     expert's per-chunk counts (in place) and its total,
//                     by wave shuffles and one barrier.
//   3. route_place    one workgroup per chunk: padded bin offsets, then the
//                     rank of each assignment among the chunk's earlier
//                     assignments to the same expert, found with wave64
//                     ballots on the expert id bits.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace bsg {

// Device memory of the allocation-free routing entry point: the per-chunk
// expert counts that bsg_route keeps in the caller's workspace.  One copy
// per GPU, held until the process ends; its host-side name is no device
// address, so host code uses only the address hipGetSymbolAddress returns
// for the device (route_scratch below).
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

hipError_t route_scratch(hipStream_t stream, int32_t** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    // the null stream runs on the current device
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // once per device, with that device current
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        addr[dev] = p;
    }
    *out = (int32_t*)addr[dev];
    return hipSuccess;
}

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kTopkThreads = 1024;                       // one workgroup per 64-token chunk
constexpr int kTopkWaves = kTopkThreads / kWave;         // 16
constexpr int kTokPerWave = kRouteChunk / kTopkWaves;    // 4 tokens per wave

// NV = logits per lane (E <= 64 NV).  Each wave first loads the logits of
// all its tokens, so the loads overlap one another, then works through them.
template <int NV>
__global__ __launch_bounds__(kTopkThreads) void route_topk(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    int32_t* __restrict__ expert_idx, float* __restrict__ gate,
    int32_t* __restrict__ chunk_counts, int nchunks) {
    __shared__ int hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kTopkThreads) hist[e] = 0;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteChunk + wave * kTokPerWave;

    float v[kTokPerWave][NV];
#pragma unroll
    for (int u = 0; u < kTokPerWave; ++u) {
        const int64_t t = t0 + u;
        const float* row = logits + t * E;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + kWave * i;
            v[u][i] = (t < T && e < E) ? row[e] : 0.0f;
        }
    }
    __syncthreads();  // histogram cleared

#pragma unroll
    for (int u = 0; u < kTokPerWave; ++u) {
        const int64_t t = t0 + u;
        if (t >= T) break;
        uint32_t taken = 0;  // bit i: expert lane + 64 i already picked
        int my_sel = -1;
        float my_val = 0.0f;
        float top_val = 0.0f;
        for (int j = 0; j < k; ++j) {
            // lane-local best among untaken experts: larger logit, then lower id
            int bi = -1;
            float bv = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = lane + kWave * i;
                if (e < E && !((taken >> i) & 1u) && (bi < 0 || v[u][i] > bv)) {
                    bi = e;
                    bv = v[u][i];
                }
            }
            // butterfly: a total order, so every lane ends with the same winner
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
                    bi = oi;
                    bv = ov;
                }
            }
            if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
            if (lane == j) {
                my_sel = bi;
                my_val = bv;
            }
            if (j == 0) top_val = bv;
        }
        // softmax over all experts, max-subtracted (the first pick is the max)
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + kWave * i;
            if (e < E) z += expf(v[u][i] - top_val);
        }
        z = wave_sum(z);
        const float p = lane < k ? expf(my_val - top_val) : 0.0f;
        const float denom = renorm ? wave_sum(p) : z;
        if (lane < k) {
            expert_idx[t * k + lane] = my_sel;
            gate[t * k + lane] = p / denom;
            atomicAdd(&hist[my_sel], 1);  // LDS only: the count is order-free
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTopkThreads)
        chunk_counts[(int64_t)e * nchunks + blockIdx.x] = hist[e];
}

// E <= 64, k <= 16: a wave's 4 tokens side by side, 16 lanes each (lane s of
// a token's segment holds experts s, s + 16, ...), so the top-k and softmax
// reductions are 4-step butterflies within 16 lanes that serve all 4 tokens
// at once.  Same selection order (larger logit, then lower id) as route_topk.
template <int NV>
__global__ __launch_bounds__(kTopkThreads) void route_topk_seg(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    int32_t* __restrict__ expert_idx, float* __restrict__ gate,
    int32_t* __restrict__ chunk_counts, int nchunks) {
    constexpr int kSeg = 16;
    static_assert(kTokPerWave * kSeg == kWave, "the wave's tokens fill its lanes");
    __shared__ int hist[kSeg * NV];
    for (int e = threadIdx.x; e < E; e += kTopkThreads) hist[e] = 0;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int sl = lane & (kSeg - 1);
    const int64_t t = (int64_t)blockIdx.x * kRouteChunk + wave * kTokPerWave + lane / kSeg;
    const bool live = t < T;

    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = sl + kSeg * i;
        v[i] = (live && e < E) ? logits[t * E + e] : 0.0f;
    }
    __syncthreads();  // histogram cleared

    uint32_t taken = 0;  // bit i: expert sl + 16 i already picked
    int my_sel = -1;
    float my_val = 0.0f;
    float top_val = 0.0f;
    for (int j = 0; j < k; ++j) {
        // lane-local best among untaken experts: larger logit, then lower id
        int bi = -1;
        float bv = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = sl + kSeg * i;
            if (e < E && !((taken >> i) & 1u) && (bi < 0 || v[i] > bv)) {
                bi = e;
                bv = v[i];
            }
        }
        // butterfly within the segment: a total order, every lane ends with the winner
#pragma unroll
        for (int off = kSeg / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kSeg);
            const int oi = __shfl_xor(bi, off, kSeg);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
                bi = oi;
                bv = ov;
            }
        }
        if ((bi & (kSeg - 1)) == sl) taken |= 1u << (bi / kSeg);
        if (sl == j) {
            my_sel = bi;
            my_val = bv;
        }
        if (j == 0) top_val = bv;
    }
    // softmax over all experts, max-subtracted (the first pick is the max)
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = sl + kSeg * i;
        if (e < E) z += expf(v[i] - top_val);
    }
#pragma unroll
    for (int off = kSeg / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, kSeg);
    const float p = sl < k ? expf(my_val - top_val) : 0.0f;
    float denom = z;
    if (renorm) {
        float ps = p;
#pragma unroll
        for (int off = kSeg / 2; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, kSeg);
        denom = ps;
    }
    if (live && sl < k) {
        expert_idx[t * k + sl] = my_sel;
        gate[t * k + sl] = p / denom;
        atomicAdd(&hist[my_sel], 1);  // LDS only: the count is order-free
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTopkThreads)
        chunk_counts[(int64_t)e * nchunks + blockIdx.x] = hist[e];
}

// Exclusive scan of one expert's chunk counts, in place; total -> counts[e].
__global__ __launch_bounds__(kRouteThreads) void route_scan(int32_t* __restrict__ chunk_counts,
                                                            int nchunks,
                                                            int32_t* __restrict__ counts) {
    __shared__ int wsum[kRouteWaves];
    int32_t* row = chunk_counts + (int64_t)blockIdx.x * nchunks;
    const int per = (nchunks + kRouteThreads - 1) / kRouteThreads;
    const int lo = threadIdx.x * per;
    const int hi = min(lo + per, nchunks);
    int s = 0;
    for (int c = lo; c < hi; ++c) s += row[c];
    int total;
    int run = block_excl_scan<kRouteWaves>(s, wsum, total);  // exclusive prefix of this segment
    for (int c = lo; c < hi; ++c) {
        const int v = row[c];
        row[c] = run;
        run += v;
    }
    if (threadIdx.x == kRouteThreads - 1) counts[blockIdx.x] = total;
}

// Bin offsets + stable in-chunk ranks -> dest_row.
__global__ __launch_bounds__(kRouteThreads) void route_place(
    const int32_t* __restrict__ expert_idx, int64_t T, int E, int k,
    const int32_t* __restrict__ chunk_base, int nchunks, const int32_t* __restrict__ counts,
    int bin_rows, int32_t* __restrict__ dest_row, int32_t* __restrict__ bin_offsets) {
    __shared__ int bins[kMaxExperts + 1];
    __shared__ int wsum[kRouteWaves];
    __shared__ int running[kMaxExperts];
    __shared__ int wcnt[kRouteWaves][kMaxExperts];

    // padded sizes, exclusive scan over ascending expert id
    const int per = (E + kRouteThreads - 1) / kRouteThreads;
    const int lo = threadIdx.x * per;
    const int hi = min(lo + per, E);
    int s = 0;
    for (int e = lo; e < hi; ++e) s += (counts[e] + bin_rows - 1) / bin_rows * bin_rows;
    for (int e = threadIdx.x; e < E; e += kRouteThreads) running[e] = 0;
    int total;
    int run = block_excl_scan<kRouteWaves>(s, wsum, total);
    for (int e = lo; e < hi; ++e) {
        bins[e] = run;
        run += (counts[e] + bin_rows - 1) / bin_rows * bin_rows;
    }
    if (threadIdx.x == kRouteThreads - 1) bins[E] = total;
    __syncthreads();
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= E; e += kRouteThreads) bin_offsets[e] = bins[e];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const int64_t a0 = (int64_t)blockIdx.x * kRouteChunk * k;
    const int64_t a1 = min(a0 + (int64_t)kRouteChunk * k, T * k);

    for (int64_t base = a0; base < a1; base += kRouteThreads) {
        for (int i = threadIdx.x; i < kRouteWaves * E; i += kRouteThreads)
            (&wcnt[0][0])[(i / E) * kMaxExperts + i % E] = 0;
        __syncthreads();
        const int64_t a = base + threadIdx.x;
        const bool valid = a < a1;
        const int e = valid ? expert_idx[a] : 0;
        // lanes of this wave holding the same expert id
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            match &= ((e >> b) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(match & lanemask_lt());
        if (valid && rank == 0) wcnt[wave][e] = __popcll(match);
        __syncthreads();
        if (valid) {
            int off = running[e];
            for (int w = 0; w < wave; ++w) off += wcnt[w][e];
            dest_row[a] = bins[e] + chunk_base[(int64_t)e * nchunks + blockIdx.x] + off + rank;
        }
        __syncthreads();
        for (int x = threadIdx.x; x < E; x += kRouteThreads) {
            int add = 0;
            for (int w = 0; w < kRouteWaves; ++w) add += wcnt[w][x];
            running[x] += add;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ gate backward
//
// The gradient of <dy, y> with respect to the logits, the top-k selection
// held fixed (plain calculus on the gate above).  One wavefront per token:
//   dg_j   = <dy[t], yp[dest_row[t*k + j]]>        (fp32, lanes over d)
//   dL/dp  = dg_j at e_j, or dg_j / S - (sum_i dg_i p[e_i]) / S^2 when the
//            gates were renormalised (S = sum_i p[e_i])
//   dlogits[t, e] = p[e] * (dL/dp[e] - sum_u p[u] dL/dp[u])
template <int NV, int DY, int YP>
__global__ __launch_bounds__(kRouteThreads) void route_backward_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ dest_row,
    const char* __restrict__ dy, int d, const char* __restrict__ yp, int64_t ld_yp_bytes,
    float* __restrict__ dlogits) {
    constexpr int DYE = DY == kBf16 ? 2 : 4, YPE = YP == kBf16 ? 2 : 4;
    constexpr int V = 16 / (DYE > YPE ? DYE : YPE);  // values per lane and step
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kRouteWaves;
    for (int64_t t = (int64_t)blockIdx.x * kRouteWaves + threadIdx.x / kWave; t < T;
         t += nwaves) {
        // ---- dg_j, kept by lane j
        float my_dg = 0.0f;
        int my_e = 0;
        for (int j = 0; j < k; ++j) {
            const int64_t row = dest_row[t * k + j];
            const char* yr = yp + row * ld_yp_bytes;
            const char* dr = dy + t * (int64_t)d * DYE;
            float s = 0.0f;
            for (int c = lane * V; c < d; c += kWave * V) {
#pragma unroll
                for (int q = 0; q < V; ++q) {
                    float a, b;
                    if constexpr (DY == kBf16) a = bf16_to_f32(((const uint16_t*)dr)[c + q]);
                    else a = ((const float*)dr)[c + q];
                    if constexpr (YP == kBf16) b = bf16_to_f32(((const uint16_t*)yr)[c + q]);
                    else b = ((const float*)yr)[c + q];
                    s = fmaf(a, b, s);
                }
            }
            s = wave_sum(s);
            if (lane == j) {
                my_dg = s;
                my_e = expert_idx[t * k + j];
            }
        }
        gate_grad_token<NV>(logits + t * E, E, k, renorm, my_dg, my_e, dlogits + t * E);
    }
}

hipError_t launch_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                                 const int32_t* expert_idx, const int32_t* dest_row,
                                 const void* dy, int dy_dtype, int d, const void* yp,
                                 int yp_dtype, int64_t ld_yp, float* dlogits,
                                 hipStream_t stream) {
    int64_t g = (T + kRouteWaves - 1) / kRouteWaves;
    const int grid = (int)(g < 8192 ? g : 8192);
    const int64_t ldb = ld_yp * (yp_dtype == kBf16 ? 2 : 4);
#define BSG_RB(NV, DY, YP)                                                                      \
    hipLaunchKernelGGL((route_backward_kernel<NV, DY, YP>), dim3(grid), dim3(kRouteThreads), 0,  \
                       stream, logits, T, E, k, renorm, expert_idx, dest_row, (const char*)dy, d, \
                       (const char*)yp, ldb, dlogits)
#define BSG_RB_NV(DY, YP)                                                                       \
    if (E <= 64) BSG_RB(1, DY, YP);                                                              \
    else if (E <= 128) BSG_RB(2, DY, YP);                                                        \
    else if (E <= 256) BSG_RB(4, DY, YP);                                                        \
    else if (E <= 512) BSG_RB(8, DY, YP);                                                        \
    else BSG_RB(16, DY, YP);
    if (dy_dtype == kBf16 && yp_dtype == kBf16) { BSG_RB_NV(kBf16, kBf16) }
    else if (dy_dtype == kBf16) { BSG_RB_NV(kBf16, kF32) }
    else if (yp_dtype == kBf16) { BSG_RB_NV(kF32, kBf16) }
    else { BSG_RB_NV(kF32, kF32) }
#undef BSG_RB_NV
#undef BSG_RB
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renorm, int bin_rows,
                        int32_t* expert_idx, float* gate, int32_t* dest_row, int32_t* counts,
                        int32_t* bin_offsets, int32_t* workspace, hipStream_t stream) {
    const int nchunks = (int)((T + kRouteChunk - 1) / kRouteChunk);
#define BSG_TOPK(NV)                                                                         \
    hipLaunchKernelGGL(route_topk<NV>, dim3(nchunks), dim3(kTopkThreads), 0, stream, logits, T, \
                       E, k, renorm, expert_idx, gate, workspace, nchunks)
#define BSG_TOPK_SEG(NV)                                                                     \
    hipLaunchKernelGGL(route_topk_seg<NV>, dim3(nchunks), dim3(kTopkThreads), 0, stream, logits, \
                       T, E, k, renorm, expert_idx, gate, workspace, nchunks)
    if (E <= 16 && k <= 16) BSG_TOPK_SEG(1);
    else if (E <= 32 && k <= 16) BSG_TOPK_SEG(2);
    else if (E <= 64 && k <= 16) BSG_TOPK_SEG(4);
    else if (E <= 64) BSG_TOPK(1);
    else if (E <= 128) BSG_TOPK(2);
    else if (E <= 256) BSG_TOPK(4);
    else if (E <= 512) BSG_TOPK(8);
    else BSG_TOPK(16);
#undef BSG_TOPK_SEG
#undef BSG_TOPK
    hipLaunchKernelGGL(route_scan, dim3(E), dim3(kRouteThreads), 0, stream, workspace, nchunks,
                       counts);
    hipLaunchKernelGGL(route_place, dim3(nchunks), dim3(kRouteThreads), 0, stream, expert_idx, T,
                       E, k, workspace, nchunks, counts, bin_rows, dest_row, bin_offsets);
    return hipGetLastError();
}

}  // namespace bsg
