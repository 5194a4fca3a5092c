// Data movement: the fused permutation + padding gather, the weighted
// un-permute/combine, and the backward's permutation of dy fused with the
// gate backward.
//
// permute_pad follows George Lin's Blog (MegaBlocks/FlexMoE post),
// section 1.4: one kernel reorders tokens from batch order into expert
// order AND pads each expert group to the 128 block size (section 1.3,
// "block size"), so the padding costs no extra pass.  unpermute_combine is
// the reverse layout transform (restore batch order) fused with the
// gate-weighted sum of each token's k expert outputs.
//
// Both are HBM-bound.  A wavefront owns one row at a time and moves it with
// 16-byte vector accesses, so every row transfer is a run of fully
// coalesced 1 KiB wave accesses.  permute_pad reads each token row ONCE and
// writes it to its k destinations.
#include "common.hpp"
#include "kernels.hpp"

namespace bsg {

constexpr int kMoveThreads = 256;
constexpr int kMoveWaves = kMoveThreads / kWave;

template <int DT>
struct Row;  // 16-byte vector of a row: 8 bf16 or 4 fp32

template <>
struct Row<kBf16> {
    static constexpr int kVec = 8;
    static __device__ __forceinline__ void load_f32(const void* p, float* out) {
        const u32x4 v = *(const u32x4*)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store_f32(void* p, const float* in) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
        *(u32x4*)p = v;
    }
};

template <>
struct Row<kF32> {
    static constexpr int kVec = 4;
    static __device__ __forceinline__ void load_f32(const void* p, float* out) {
        const f32x4 v = *(const f32x4*)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = v[i];
    }
    static __device__ __forceinline__ void store_f32(void* p, const float* in) {
        *(f32x4*)p = f32x4{in[0], in[1], in[2], in[3]};
    }
};

// Scaled copy of one 16-byte chunk: each product rounded once.
template <int DT>
__device__ __forceinline__ u32x4 scale_chunk(u32x4 v, float s);

// bf16(s * v) rounded once, without fp64 in the common case: p = fl(s v)
// and its exact error e = s v - p (one FMA) give the product rounded to
// odd at fp32 precision (truncate towards zero, set the last bit when
// inexact), and rounding that to bf16 equals rounding s v itself, since
// fp32 keeps more than two bits beyond bf16's.  Products too small or too
// large for e to be exact, zeros and non-finite values take the fp64 path.
__device__ __forceinline__ uint32_t scaled_bf16(float s, float v) {
    const float p = s * v;
    const float ap = fabsf(p);
    if (!(ap >= 0x1p-100f) || !(ap <= 0x1p+100f)) return f64_to_bf16((double)s * (double)v);
    const float e = fmaf(s, v, -p);
    uint32_t u = __float_as_uint(p);
    if (e != 0.0f) {
        if ((e < 0.0f) != (p < 0.0f)) u -= 1u;  // |s v| < |p|: step towards zero
        u |= 1u;
    }
    return f32_to_bf16(__uint_as_float(u));
}

template <>
__device__ __forceinline__ u32x4 scale_chunk<kBf16>(u32x4 v, float s) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = scaled_bf16(s, __uint_as_float(v[i] << 16));
        const uint32_t hi = scaled_bf16(s, __uint_as_float(v[i] & 0xffff0000u));
        o[i] = lo | (hi << 16);
    }
    return o;
}

template <>
__device__ __forceinline__ u32x4 scale_chunk<kF32>(u32x4 v, float s) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = __float_as_uint((float)((double)s * (double)__uint_as_float(v[i])));
    return o;
}

// Jobs: token rows [0, T) then pad slots [T, T + E*128).  A pad slot (e, i)
// is row bin_offsets[e] + counts[e] + i when that row is still in e's bin.
template <int DT>
__global__ __launch_bounds__(kMoveThreads) void permute_pad_kernel(
    const u32x4* __restrict__ x, int64_t T, int chunks, int k, const int32_t* __restrict__ dest_row,
    const float* __restrict__ scale, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ bin_offsets, int E, int bin_rows, int64_t Tp_max,
    int32_t* __restrict__ row_src, u32x4* __restrict__ xp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kMoveWaves;
    const int64_t njobs = T + (int64_t)E * bin_rows;  // a bin's tail is below bin_rows rows
    for (int64_t job = (int64_t)blockIdx.x * kMoveWaves + threadIdx.x / kWave; job < njobs;
         job += nwaves) {
        if (job < T) {
            const int64_t t = job;
            const u32x4* src = x + t * chunks;
            for (int c = lane; c < chunks; c += kWave) {
                const u32x4 v = src[c];
                for (int j = 0; j < k; ++j) {
                    const int64_t a = t * k + j;
                    const int64_t row = dest_row[a];
                    if (row < Tp_max)  // holds whenever the routing used this bin size
                        xp[row * chunks + c] = scale ? scale_chunk<DT>(v, scale[a]) : v;
                }
            }
            if (lane < k && dest_row[t * k + lane] < Tp_max)
                row_src[dest_row[t * k + lane]] = (int32_t)(t * k + lane);
        } else {
            const int64_t p = job - T;
            const int e = (int)(p / bin_rows);
            const int64_t row = (int64_t)bin_offsets[e] + counts[e] + p % bin_rows;
            if (row >= bin_offsets[e + 1] || row >= Tp_max) continue;
            u32x4* dst = xp + row * chunks;
            for (int c = lane; c < chunks; c += kWave) dst[c] = u32x4{0u, 0u, 0u, 0u};
            if (lane == 0) row_src[row] = -1;
        }
    }
}

// The backward's first step in one pass over dy: dYp = permute_pad(dy,
// scale = gate), exactly as permute_pad_kernel, and the gate backward of
// each token: dg_j = <dy_t, yp_j> accumulated (fp32) while dy's chunks are
// in registers, then the router-logit gradient (gate_grad_token).
//
// PAIR: rows of at least two wave-widths of chunks keep two chunks per lane
// in flight; shorter rows take one chunk per step, which needs fewer
// registers (more waves per SIMD).
template <int DT, int YP, int NV, bool PAIR>
__global__ __launch_bounds__(kMoveThreads) void permute_gate_backward_kernel(
    const u32x4* __restrict__ dy, int64_t T, int chunks, int k,
    const int32_t* __restrict__ dest_row, const float* __restrict__ gate,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ bin_offsets, int E,
    int bin_rows, int64_t Tp_max, int32_t* __restrict__ row_src, u32x4* __restrict__ dyp,
    const float* __restrict__ logits, int renorm, const int32_t* __restrict__ expert_idx,
    const char* __restrict__ yp, int64_t ld_yp_bytes, float* __restrict__ dlogits) {
    constexpr int V = Row<DT>::kVec;                       // dy values per 16-byte chunk
    constexpr int YCB = V * (YP == kBf16 ? 2 : 4);         // yp bytes of those values
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kMoveWaves;
    const int64_t njobs = T + (int64_t)E * bin_rows;
    for (int64_t job = (int64_t)blockIdx.x * kMoveWaves + threadIdx.x / kWave; job < njobs;
         job += nwaves) {
        if (job < T) {
            const int64_t t = job;
            const u32x4* src = dy + t * chunks;
            // the token's picks (and, for long rows, its logits) are
            // requested first, so the softmax at the end waits on nothing
            float lg[NV];
            if constexpr (PAIR) load_logits<NV>(logits + t * E, E, lg);
            const int my_e = lane < k ? expert_idx[t * k + lane] : 0;
            float my_dg = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int64_t a = t * k + j;
                const int64_t row = dest_row[a];
                const float g = gate[a];
                const char* yr = yp + row * ld_yp_bytes;
                float s = 0.0f;
                if constexpr (PAIR) {
                    // two chunks per lane in flight; row < Tp_max whenever
                    // the routing used this bin size
                    for (int c0 = lane; c0 < chunks && row < Tp_max; c0 += 2 * kWave) {
                        const int c1 = c0 + kWave;
                        const bool two = c1 < chunks;
                        // raw 16-byte words in flight (yp: YCB / 16 words a chunk)
                        u32x4 v[2], w[2][YCB / 16];
                        v[0] = src[c0];
                        if (two) v[1] = src[c1];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            if (h == 1 && !two) break;
                            const int c = h == 0 ? c0 : c1;
#pragma unroll
                            for (int u = 0; u < YCB / 16; ++u)
                                w[h][u] = *(const u32x4*)(yr + (int64_t)c * YCB + 16 * u);
                        }
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            if (h == 1 && !two) break;
                            const int c = h == 0 ? c0 : c1;
                            dyp[row * chunks + c] = scale_chunk<DT>(v[h], g);
                            float x[V], y[V];
                            Row<DT>::load_f32(&v[h], x);
                            if constexpr (YCB == 16) {
                                Row<YP>::load_f32(&w[h][0], y);
                            } else {  // bf16 dy, fp32 yp: two 16-byte words of yp
                                Row<kF32>::load_f32(&w[h][0], y);
                                Row<kF32>::load_f32(&w[h][1], y + 4);
                            }
#pragma unroll
                            for (int q = 0; q < V; ++q) s = fmaf(x[q], y[q], s);
                        }
                    }
                } else {
                    for (int c = lane; c < chunks && row < Tp_max; c += kWave) {
                        const u32x4 v = src[c];
                        dyp[row * chunks + c] = scale_chunk<DT>(v, g);
                        float x[V], y[V];
                        Row<DT>::load_f32(&v, x);
                        if constexpr (YCB == 16) {
                            Row<YP>::load_f32(yr + (int64_t)c * 16, y);
                        } else {  // bf16 dy, fp32 yp: two 16-byte chunks of yp
                            Row<kF32>::load_f32(yr + (int64_t)c * 32, y);
                            Row<kF32>::load_f32(yr + (int64_t)c * 32 + 16, y + 4);
                        }
#pragma unroll
                        for (int q = 0; q < V; ++q) s = fmaf(x[q], y[q], s);
                    }
                }
                s = wave_sum(s);
                if (lane == j) my_dg = s;
            }
            if (lane < k && dest_row[t * k + lane] < Tp_max)
                row_src[dest_row[t * k + lane]] = (int32_t)(t * k + lane);
            if constexpr (!PAIR) load_logits<NV>(logits + t * E, E, lg);
            gate_grad_token_loaded<NV>(lg, E, k, renorm, my_dg, my_e, dlogits + t * E);
        } else {
            const int64_t p = job - T;
            const int e = (int)(p / bin_rows);
            const int64_t row = (int64_t)bin_offsets[e] + counts[e] + p % bin_rows;
            if (row >= bin_offsets[e + 1] || row >= Tp_max) continue;
            u32x4* dst = dyp + row * chunks;
            for (int c = lane; c < chunks; c += kWave) dst[c] = u32x4{0u, 0u, 0u, 0u};
            if (lane == 0) row_src[row] = -1;
        }
    }
}

// y[t] = sum_j g_j * yp[dest_row[t*k + j]], fp32 accumulation in ascending j.
template <int DT_IN, int DT_OUT>
__global__ __launch_bounds__(kMoveThreads) void combine_kernel(
    const char* __restrict__ yp, int64_t ld_yp_bytes, const int32_t* __restrict__ dest_row,
    const float* __restrict__ gate, int64_t T, int k, int d, char* __restrict__ y) {
    constexpr int V = Row<DT_IN>::kVec;
    constexpr int ES_IN = DT_IN == kBf16 ? 2 : 4;
    constexpr int ES_OUT = DT_OUT == kBf16 ? 2 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kMoveWaves;
    const int groups = d / V;
    for (int64_t t = (int64_t)blockIdx.x * kMoveWaves + threadIdx.x / kWave; t < T; t += nwaves) {
        for (int c = lane; c < groups; c += kWave) {
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int64_t a = t * k + j;
                const float g = gate ? gate[a] : 1.0f;
                float v[V];
                Row<DT_IN>::load_f32(yp + (int64_t)dest_row[a] * ld_yp_bytes +
                                         (int64_t)c * V * ES_IN, v);
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] += g * v[i];
            }
            char* dst = y + (t * d + (int64_t)c * V) * ES_OUT;
            if constexpr (ES_OUT * V == 16) {
                Row<DT_OUT>::store_f32(dst, acc);  // same width in and out
            } else if constexpr (DT_OUT == kBf16) {  // 4 fp32 in -> 4 bf16 = 8 bytes
                *(u32x2*)dst = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            } else {  // 8 bf16 in -> 8 fp32 out = two 16-byte stores
                Row<kF32>::store_f32(dst, acc);
                Row<kF32>::store_f32(dst + 16, acc + 4);
            }
        }
    }
}

// A plain streaming copy of n 16-byte words, the HBM ceiling the
// data-movement calls are measured against: every word read once and
// written once.  Two forms, the faster of a sweep on the MI355X (grid sizes
// 1K-64K workgroups, 2-16 words in flight per thread, temporal and
// non-temporal accesses): up to 512 MiB, a grid-stride loop over up to
// 16384 workgroups with eight loads of each thread in flight (4.1 TB/s at
// 53 MB, 5.25 TB/s at 200 MB);
// beyond it, each workgroup copies 16 KB blocks, four words per thread
// (5.6 TB/s at 1 GiB).
__global__ __launch_bounds__(kMoveThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t n) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * kMoveThreads;
    int64_t i = (int64_t)blockIdx.x * kMoveThreads + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kMoveThreads) void stream_copy_blocks_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
    constexpr int U = 4;
    constexpr int64_t kChunk = (int64_t)kMoveThreads * U;
    for (int64_t base = (int64_t)blockIdx.x * kChunk; base < n; base += (int64_t)gridDim.x * kChunk) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + u * kMoveThreads + threadIdx.x;
            if (j < n) v[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + u * kMoveThreads + threadIdx.x;
            if (j < n) dst[j] = v[u];
        }
    }
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    if (words * 16 > (int64_t(512) << 20)) {
        const int64_t chunks = (words + kMoveThreads * 4 - 1) / (kMoveThreads * 4);
        const int grid = (int)(chunks < 65536 ? chunks : 65536);
        hipLaunchKernelGGL(stream_copy_blocks_kernel, dim3(grid), dim3(kMoveThreads), 0, stream,
                           (const u32x4*)src, (u32x4*)dst, words);
    } else {
        // as many workgroups as the sweep found best: up to 16384, never more
        // than one word per thread
        const int64_t g = (words + kMoveThreads - 1) / kMoveThreads;
        const int grid = (int)(g < 16384 ? g : 16384);
        hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(kMoveThreads), 0, stream,
                           (const u32x4*)src, (u32x4*)dst, words);
    }
    return hipGetLastError();
}

static int move_grid(int64_t jobs) {
    int64_t g = (jobs + kMoveWaves - 1) / kMoveWaves;
    return (int)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

hipError_t launch_permute_pad(const void* x, int dtype, int64_t T, int d, int k,
                              const int32_t* dest_row, const float* scale, const int32_t* counts,
                              const int32_t* bin_offsets, int E, int bin_rows, int64_t Tp_max,
                              int32_t* row_src, void* xp, hipStream_t stream) {
    const int es = dtype == kBf16 ? 2 : 4;
    const int chunks = d * es / 16;
    const int grid = move_grid(T + (int64_t)E * bin_rows);
    if (dtype == kBf16)
        hipLaunchKernelGGL(permute_pad_kernel<kBf16>, dim3(grid), dim3(kMoveThreads), 0, stream,
                           (const u32x4*)x, T, chunks, k, dest_row, scale, counts, bin_offsets, E,
                           bin_rows, Tp_max, row_src, (u32x4*)xp);
    else
        hipLaunchKernelGGL(permute_pad_kernel<kF32>, dim3(grid), dim3(kMoveThreads), 0, stream,
                           (const u32x4*)x, T, chunks, k, dest_row, scale, counts, bin_offsets, E,
                           bin_rows, Tp_max, row_src, (u32x4*)xp);
    return hipGetLastError();
}

template <int DT, int YP>
static hipError_t launch_pgb(const void* dy, int64_t T, int d, int k, const int32_t* dest_row,
                             const float* gate, const int32_t* counts,
                             const int32_t* bin_offsets, int E, int bin_rows, int64_t Tp_max,
                             int32_t* row_src, void* dyp, const float* logits, int renorm,
                             const int32_t* expert_idx, const void* yp, int64_t ld_yp_bytes,
                             float* dlogits, hipStream_t stream) {
    const int chunks = d * (DT == kBf16 ? 2 : 4) / 16;
    const int grid = move_grid(T + (int64_t)E * bin_rows);
#define BSG_PGB(NV, PAIR)                                                                        \
    hipLaunchKernelGGL((permute_gate_backward_kernel<DT, YP, NV, PAIR>), dim3(grid),             \
                       dim3(kMoveThreads), 0, stream, (const u32x4*)dy, T, chunks, k, dest_row,  \
                       gate, counts, bin_offsets, E, bin_rows, Tp_max, row_src, (u32x4*)dyp,     \
                       logits, renorm, expert_idx, (const char*)yp, ld_yp_bytes, dlogits)
#define BSG_PGB_E(PAIR)                   \
    if (E <= 64) BSG_PGB(1, PAIR);        \
    else if (E <= 128) BSG_PGB(2, PAIR);  \
    else if (E <= 256) BSG_PGB(4, PAIR);  \
    else if (E <= 512) BSG_PGB(8, PAIR);  \
    else BSG_PGB(16, PAIR);
    if (chunks >= 2 * kWave) {
        BSG_PGB_E(true)
    } else {
        BSG_PGB_E(false)
    }
#undef BSG_PGB_E
#undef BSG_PGB
    return hipGetLastError();
}

hipError_t launch_permute_gate_backward(const void* dy, int dtype, int64_t T, int d, int k,
                                        const int32_t* dest_row, const float* gate,
                                        const int32_t* counts, const int32_t* bin_offsets, int E,
                                        int bin_rows, int64_t Tp_max, int32_t* row_src,
                                        void* dyp,
                                        const float* logits, int renorm,
                                        const int32_t* expert_idx, const void* yp, int yp_dtype,
                                        int64_t ld_yp, float* dlogits, hipStream_t stream) {
    const int64_t ldb = ld_yp * (yp_dtype == kBf16 ? 2 : 4);
    if (dtype == kBf16 && yp_dtype == kBf16)
        return launch_pgb<kBf16, kBf16>(dy, T, d, k, dest_row, gate, counts, bin_offsets, E,
                                        bin_rows, Tp_max, row_src, dyp, logits, renorm, expert_idx, yp,
                                        ldb, dlogits, stream);
    if (dtype == kBf16)
        return launch_pgb<kBf16, kF32>(dy, T, d, k, dest_row, gate, counts, bin_offsets, E,
                                       bin_rows, Tp_max, row_src, dyp, logits, renorm, expert_idx, yp,
                                       ldb, dlogits, stream);
    if (yp_dtype == kF32)
        return launch_pgb<kF32, kF32>(dy, T, d, k, dest_row, gate, counts, bin_offsets, E,
                                      bin_rows, Tp_max, row_src, dyp, logits, renorm, expert_idx, yp, ldb,
                                      dlogits, stream);
    return hipErrorInvalidValue;  // fp32 dy with bf16 yp: not a layout the layer produces
}

hipError_t launch_unpermute_combine(const void* yp, int yp_dtype, int64_t ld_yp,
                                    const int32_t* dest_row, const float* gate, int64_t T, int k,
                                    int d, void* y, int y_dtype, hipStream_t stream) {
    const int grid = move_grid(T);
    const int64_t ldb = ld_yp * (yp_dtype == kBf16 ? 2 : 4);
#define BSG_COMBINE(I, O)                                                                        \
    hipLaunchKernelGGL((combine_kernel<I, O>), dim3(grid), dim3(kMoveThreads), 0, stream,        \
                       (const char*)yp, ldb, dest_row, gate, T, k, d, (char*)y)
    if (yp_dtype == kBf16 && y_dtype == kBf16) BSG_COMBINE(kBf16, kBf16);
    else if (yp_dtype == kBf16) BSG_COMBINE(kBf16, kF32);
    else if (y_dtype == kBf16) BSG_COMBINE(kF32, kBf16);
    else BSG_COMBINE(kF32, kF32);
#undef BSG_COMBINE
    return hipGetLastError();
}

}  // namespace bsg
