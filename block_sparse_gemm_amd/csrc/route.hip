// Routing: gate + router, histogram, padded bins and stable placement.
//
// George Lin's Blog (MegaBlocks/FlexMoE post), section 1.4: tokens are
// routed to experts and regrouped from batch order into expert order, each
// group padded to a multiple of the 128 block size (section 1.3), or of a
// finer or coarser bin (64 or 256 rows) for the block-size study.  The
// pages leave the gate's form open; this follows top-k on the logits with a
// softmax gate.
//
// Two launches, no atomics on global memory, so every integer result is
// identical on every run:
//   1. route_topk     one workgroup per 64-token chunk, one wavefront per
//                     token at a time (4 each, loaded up front): top-k by
//                     wave reductions, softmax gate; an LDS histogram, the
//                     chunk's row of a chunk-major count matrix.  Up to 64
//                     experts and top-16 (route_topk_seg): the 4 tokens of a
//                     wave side by side, 16 lanes each.
//   2. route_place    one workgroup per 16 chunks: every workgroup sums the
//                     count matrix (per-expert totals, and the counts of the
//                     chunks before its own), forms the padded bin offsets,
//                     then ranks each of its assignments among the earlier
//                     ones of the same expert with wave64 ballots on the
//                     expert id bits.  It can also write the topology of
//                     those bins (topology.hpp), so route + topology is two
//                     launches.
// Routings too large for every workgroup to read the whole count matrix
// scan it first in a launch of its own (route_scan, one workgroup per
// expert).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"
#include "topology.hpp"

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
    int32_t* __restrict__ chunk_counts) {
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
        chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// E <= 64, k <= 16: a wave's 4 tokens side by side, 16 lanes each (lane s of
// a token's segment holds experts s, s + 16, ...), so the top-k and softmax
// reductions are 4-step butterflies within 16 lanes that serve all 4 tokens
// at once.  Same selection order (larger logit, then lower id) as route_topk.
template <int NV>
__global__ __launch_bounds__(kTopkThreads) void route_topk_seg(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    int32_t* __restrict__ expert_idx, float* __restrict__ gate,
    int32_t* __restrict__ chunk_counts) {
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
        chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of one expert's chunk counts (column e of the chunk-major
// count matrix), in place; total -> counts[e].  Only for routings too large
// for the placement to sum the counts itself.
__global__ __launch_bounds__(kRouteThreads) void route_scan(int32_t* __restrict__ chunk_counts,
                                                            int nchunks, int E,
                                                            int32_t* __restrict__ counts) {
    __shared__ int wsum[kRouteWaves];
    int32_t* col = chunk_counts + blockIdx.x;
    const int per = (nchunks + kRouteThreads - 1) / kRouteThreads;
    const int lo = threadIdx.x * per;
    const int hi = min(lo + per, nchunks);
    int s = 0;
    for (int c = lo; c < hi; ++c) s += col[(int64_t)c * E];
    int total;
    int run = block_excl_scan<kRouteWaves>(s, wsum, total);  // exclusive prefix of this segment
    for (int c = lo; c < hi; ++c) {
        const int v = col[(int64_t)c * E];
        col[(int64_t)c * E] = run;
        run += v;
    }
    if (threadIdx.x == kRouteThreads - 1) counts[blockIdx.x] = total;
}

constexpr int kPlaceThreads = 1024;
constexpr int kPlaceWaves = kPlaceThreads / kWave;  // 16
constexpr int kPlaceChunks = 16;  // chunks (1024 tokens) per placing workgroup
// With the permutation in the same launch, a placing workgroup takes fewer
// chunks (so that enough workgroups copy rows), at most this many of its
// assignments, whose rows it keeps in LDS for the copy.
constexpr int kPermMax = 4096;
// Every placement workgroup sums the whole count matrix itself when it has
// at most this many entries, the routing at most this many chunks and the
// placing workgroups together read at most kSelfScanReads counts; larger
// routings scan it in a launch of their own first.
constexpr int64_t kSelfScanCounts = 65536;
constexpr int kSelfScanChunks = 1024;
constexpr int64_t kSelfScanReads = int64_t(1) << 23;

// Per-expert totals and this workgroup's starting ranks (the assignments
// of chunks before c0) from the raw chunk-major counts, into LDS (both
// cleared by the caller).  VEC: E is a power of two in [4, 1024] and the
// counts are 16-byte aligned, so a thread's 4-count vectors always hold
// the same 4 experts and it sums them in registers.
template <bool VEC>
__device__ __forceinline__ void sum_chunk_counts(const int32_t* __restrict__ cc, int nchunks,
                                                 int E, int c0, int* tot, int* pre) {
    const int64_t n = (int64_t)nchunks * E;
    if constexpr (VEC) {
        const int4* v4 = (const int4*)cc;
        const int64_t n4 = n / 4;
        const int e0 = (4 * threadIdx.x) & (E - 1);
        int t[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0};
        int64_t i = threadIdx.x;
        for (; i + 3 * kPlaceThreads < n4; i += 4 * kPlaceThreads) {
            int4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = v4[i + u * kPlaceThreads];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool before = (4 * (i + u * kPlaceThreads)) / E < c0;
                t[0] += v[u].x; t[1] += v[u].y; t[2] += v[u].z; t[3] += v[u].w;
                if (before) { p[0] += v[u].x; p[1] += v[u].y; p[2] += v[u].z; p[3] += v[u].w; }
            }
        }
        for (; i < n4; i += kPlaceThreads) {
            const int4 v = v4[i];
            t[0] += v.x; t[1] += v.y; t[2] += v.z; t[3] += v.w;
            if ((4 * i) / E < c0) { p[0] += v.x; p[1] += v.y; p[2] += v.z; p[3] += v.w; }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (t[q]) atomicAdd(&tot[e0 + q], t[q]);  // LDS only: integer sums, order-free
            if (p[q]) atomicAdd(&pre[e0 + q], p[q]);
        }
    } else {
        for (int64_t i = threadIdx.x; i < n; i += kPlaceThreads) {
            const int v = cc[i];
            if (!v) continue;
            const int e = (int)(i % E);
            atomicAdd(&tot[e], v);
            if (i / E < c0) atomicAdd(&pre[e], v);
        }
    }
}

// Counts, padded bin offsets and dest_row; with `topo.on`, also the
// topology of those bins; with PERM, also the permuted, padded copy of x.
// Every workgroup forms the bins; the first `nplace` workgroups then place,
// workgroup w the assignments of chunks [cpw w, cpw (w + 1)): the rank of
// each assignment among the earlier ones of its expert, from the count of
// the earlier chunks plus wave64 ballots on the expert id bits inside the
// workgroup.  With PERM each of them then copies its tokens' rows to their
// places and zero-fills the pad rows of experts w, w + nplace, ...  The
// workgroups after them write the topology (topology.hpp) meanwhile, so it
// costs no launch and little time of its own.  SCANNED: route_scan has
// already turned the counts into per-expert exclusive prefixes and totals;
// else each workgroup sums them itself.
template <bool SCANNED, bool VEC, bool PERM>
// Eight waves per SIMD (at most 64 VGPRs): two workgroups share a CU, so the
// whole grid (placing and topology workgroups) is resident from the start.
__global__ __launch_bounds__(kPlaceThreads) __attribute__((amdgpu_waves_per_eu(8))) void route_place(
    const int32_t* __restrict__ expert_idx, int64_t T, int E, int k,
    const int32_t* __restrict__ chunk_counts, int nchunks, int nplace, int cpw,
    int32_t* __restrict__ counts, int bin_rows, int32_t* __restrict__ dest_row,
    int32_t* __restrict__ bin_offsets, TopoJob topo, PermJob perm) {
    __shared__ int pdest[PERM ? kPermMax : 1];  // rows of this workgroup's assignments
    __shared__ int tot[kMaxExperts];
    __shared__ int running[kMaxExperts];
    __shared__ int bins[kMaxExperts + 1];
    __shared__ int2 wsum2[kPlaceWaves];
    // per wave and expert, kPlaceWaves x E (dynamic LDS: 4 KB at 64
    // experts, so two workgroups share a CU and every workgroup of the
    // launch is resident at once)
    extern __shared__ int wcnt[];
    __shared__ TopoLds<kPlaceThreads> tl;

    const bool placer = (int)blockIdx.x < nplace;
    const int c0 = placer ? (int)blockIdx.x * cpw : 0;
    const int64_t A = T * k;
    const int64_t a0 = placer ? min((int64_t)c0 * kRouteChunk * k, A) : 0;
    const int64_t a1 = placer ? min(a0 + (int64_t)cpw * kRouteChunk * k, A) : 0;
    // the first round's expert ids, loaded while the counts are summed
    const int e_first = (a0 + threadIdx.x < a1) ? expert_idx[a0 + threadIdx.x] : 0;

    if constexpr (SCANNED) {
        for (int e = threadIdx.x; e < E; e += kPlaceThreads) {
            tot[e] = counts[e];
            running[e] = placer ? chunk_counts[(int64_t)c0 * E + e] : 0;
        }
    } else {
        for (int e = threadIdx.x; e < E; e += kPlaceThreads) tot[e] = running[e] = 0;
    }
    for (int i = threadIdx.x; i < kPlaceWaves * E; i += kPlaceThreads) wcnt[i] = 0;
    if (threadIdx.x == 0) tl.misaligned = 0;
    __syncthreads();
    if constexpr (!SCANNED) {
        sum_chunk_counts<VEC>(chunk_counts, nchunks, E, c0, tot, running);
        __syncthreads();
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e < E; e += kPlaceThreads) counts[e] = tot[e];
    }

    // padded sizes, exclusive scan over ascending expert id; with a
    // topology, the same scan also counts each expert's 256-row tiles and
    // leaves the topology's LDS state (bin starts in block rows, first tile
    // of each expert) ready
    {
        const int br = topo.on ? topo.br : kBlock;
        const int per = (E + kPlaceThreads - 1) / kPlaceThreads;
        const int lo = threadIdx.x * per;
        const int hi = min(lo + per, E);
        int2 v = make_int2(0, 0);
        for (int e = lo; e < hi; ++e) {
            const int pe = (tot[e] + bin_rows - 1) / bin_rows * bin_rows;
            v.x += pe;
            v.y += (pe + 255) / 256;
        }
        int2 total;
        int2 run = block_excl_scan2<kPlaceWaves>(v, wsum2, total);
        for (int e = lo; e < hi; ++e) {
            const int pe = (tot[e] + bin_rows - 1) / bin_rows * bin_rows;
            bins[e] = run.x;
            tl.s[e] = run.x / br;
            tl.pp[e] = run.y;
            if (run.x % br) tl.misaligned = 1;  // a bin off the block grid
            run.x += pe;
            run.y += (pe + 255) / 256;
        }
        if (threadIdx.x == kPlaceThreads - 1) {
            bins[E] = total.x;
            tl.s[E] = total.x / br;
            tl.pp[E] = total.y;
            if (total.x % br) tl.misaligned = 1;
        }
        __syncthreads();
    }
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= E; e += kPlaceThreads) bin_offsets[e] = bins[e];

    if (!placer) {
        if (topo.on) {
            topo_order(tl, E, (int)((blockIdx.x - nplace) * kPlaceWaves + threadIdx.x / kWave),
                       (int)((gridDim.x - nplace) * kPlaceWaves), topo.o.expert_order);
            topo_write<kPlaceThreads>((int64_t)(blockIdx.x - nplace) * kPlaceThreads + threadIdx.x,
                                      tl, E, topo.F, topo.br, topo.row_blocks_max, topo.group,
                                      topo.o);
        }
        return;
    }

    // rounds of 1024 assignments; wcnt starts each round cleared
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int64_t base = a0; base < a1; base += kPlaceThreads) {
        const int64_t a = base + threadIdx.x;
        const bool valid = a < a1;
        const int e = base == a0 ? e_first : (valid ? expert_idx[a] : 0);
        // lanes of this wave holding the same expert id
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            match &= ((e >> b) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(match & lanemask_lt());
        if (valid && rank == 0) wcnt[wave * E + e] = __popcll(match);
        __syncthreads();
        // per expert: each wave's first rank (the expert's running count plus
        // the earlier waves' counts), in place of the counts
        for (int x = threadIdx.x; x < E; x += kPlaceThreads) {
            int run = running[x];
#pragma unroll
            for (int w = 0; w < kPlaceWaves; ++w) {
                const int c = wcnt[w * E + x];
                wcnt[w * E + x] = run;
                run += c;
            }
            running[x] = run;
        }
        __syncthreads();
        if (valid) {
            const int r = bins[e] + wcnt[wave * E + e] + rank;
            dest_row[a] = r;
            if constexpr (PERM) pdest[a - a0] = r;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < kPlaceWaves * E; i += kPlaceThreads) wcnt[i] = 0;
        __syncthreads();
    }

    if constexpr (PERM) {
        // the permuted copy: token t's row is read once and written to the
        // rows of its k assignments (the rounds above end with a barrier, so
        // pdest is complete); rows at or past Tp_max are never written
        const u32x4* __restrict__ x = (const u32x4*)perm.x;
        u32x4* __restrict__ xp = (u32x4*)perm.xp;
        const int chunks = perm.chunks;
        // each wave takes kCopyTokens tokens at a time and loads all their
        // chunks before it stores any, so several loads per lane are in
        // flight (one token at a time left the copy latency-bound)
        constexpr int kCopyTokens = 4;
        const int64_t t0 = a0 / k, t1 = a1 / k;
        for (int64_t tb = t0 + (int64_t)wave * kCopyTokens; tb < t1;
             tb += (int64_t)kPlaceWaves * kCopyTokens) {
            const int nu = (int)min((int64_t)kCopyTokens, t1 - tb);
            const int* pd = pdest + (tb - t0) * k;
            for (int c = lane; c < chunks; c += kWave) {
                u32x4 v[kCopyTokens];
#pragma unroll
                for (int u = 0; u < kCopyTokens; ++u)
                    if (u < nu) v[u] = x[(tb + u) * chunks + c];
#pragma unroll
                for (int u = 0; u < kCopyTokens; ++u) {
                    if (u >= nu) break;
                    for (int j = 0; j < k; ++j) {
                        const int64_t r = pd[u * k + j];
                        if (r < perm.Tp_max) xp[r * chunks + c] = v[u];
                    }
                }
            }
            for (int q = lane; q < nu * k; q += kWave)
                if (pd[q] < perm.Tp_max) perm.row_src[pd[q]] = (int32_t)(tb * k + q);
        }
        // the pad rows of experts blockIdx.x, + nplace, ...: zeros, row_src -1
        for (int e = blockIdx.x; e < E; e += nplace) {
            const int64_t hi = min((int64_t)bins[e + 1], perm.Tp_max);
            for (int64_t r = (int64_t)bins[e] + tot[e] + wave; r < hi; r += kPlaceWaves) {
                u32x4* dst = xp + r * chunks;
                for (int c = lane; c < chunks; c += kWave) dst[c] = u32x4{0u, 0u, 0u, 0u};
                if (lane == 0) perm.row_src[r] = -1;
            }
        }
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
                        int32_t* bin_offsets, int32_t* workspace, const TopoJob& topo,
                        const PermJob& perm, hipStream_t stream) {
    const int nchunks = (int)((T + kRouteChunk - 1) / kRouteChunk);
#define BSG_TOPK(NV)                                                                         \
    hipLaunchKernelGGL(route_topk<NV>, dim3(nchunks), dim3(kTopkThreads), 0, stream, logits, T, \
                       E, k, renorm, expert_idx, gate, workspace)
#define BSG_TOPK_SEG(NV)                                                                     \
    hipLaunchKernelGGL(route_topk_seg<NV>, dim3(nchunks), dim3(kTopkThreads), 0, stream, logits, \
                       T, E, k, renorm, expert_idx, gate, workspace)
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
    // chunks per placing workgroup: 16, or with the permutation about one
    // placing workgroup per CU (each keeps at most kPermMax rows in LDS)
    int cpw = kPlaceChunks;
    if (perm.on) {
        const int maxc = kPermMax / (kRouteChunk * k);  // >= 2: k <= 32
        cpw = std::min(maxc, std::max(1, (nchunks + 255) / 256));
    }
    // placing workgroups, then (with a topology) the topology's
    const int nplace = (nchunks + cpw - 1) / cpw;
    int64_t grid = nplace;
    if (topo.on)
        grid += (topo_threads(E, topo.F, topo.row_blocks_max, topo.row_tiles_max) +
                 kPlaceThreads - 1) / kPlaceThreads;
    const bool self_scan = (int64_t)nchunks * E <= kSelfScanCounts &&
                           nchunks <= kSelfScanChunks &&
                           (int64_t)nplace * nchunks * E <= kSelfScanReads;
    const bool vec = E >= 4 && (E & (E - 1)) == 0 && ((uintptr_t)workspace & 15) == 0;
    const size_t wcnt_bytes = (size_t)kPlaceWaves * E * sizeof(int);
#define BSG_PLACE(S, V, P)                                                                     \
    hipLaunchKernelGGL((route_place<S, V, P>), dim3(grid), dim3(kPlaceThreads), wcnt_bytes,      \
                       stream, expert_idx, T, E, k, workspace, nchunks, nplace, cpw, counts,    \
                       bin_rows, dest_row, bin_offsets, topo, perm)
    if (!self_scan)
        hipLaunchKernelGGL(route_scan, dim3(E), dim3(kRouteThreads), 0, stream, workspace,
                           nchunks, E, counts);
    if (perm.on) {
        if (!self_scan) BSG_PLACE(true, false, true);
        else if (vec) BSG_PLACE(false, true, true);
        else BSG_PLACE(false, false, true);
    } else {
        if (!self_scan) BSG_PLACE(true, false, false);
        else if (vec) BSG_PLACE(false, true, false);
        else BSG_PLACE(false, false, false);
    }
#undef BSG_PLACE
    return hipGetLastError();
}

}  // namespace bsg
