// Device-side helpers shared by the gfx950 kernels of the block-sparse
// expert layer: vector types, bf16 conversion, wave reductions, the
// XCD-aware workgroup remap and the fp32 activation functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 128;       // block edge of the sparse layout
constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (lo, hi), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950, no branches.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// fp64 -> bf16 rounded ONCE to nearest even: truncate to fp32, make the
// result sticky-odd when inexact (round to odd keeps enough bits), then
// round to nearest even into bf16.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
    float f = __double2float_rz(v);
    uint32_t u = __float_as_uint(f);
    if ((double)f != v) u |= 1u;
    return f32_to_bf16(__uint_as_float(u));
}

// ---------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ------------------------------------------------------------ XCD remap
//
// Workgroup w of an n-workgroup launch runs on XCD w % 8.  Give each XCD a
// contiguous range of logical tiles so that neighbouring tiles, which share
// operand panels, hit the same L2.  Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int w, int n) {
    const int q = n / kXcds, r = n % kXcds, x = w % kXcds, i = w / kXcds;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Chunked variant: chunks of C consecutive tiles are dealt to the XCDs in
// turn, so tiles early in the order start first on every XCD (the order is
// kept across the chip) while each chunk stays in one XCD's L2.  The tail
// that does not fill a round falls back to xcd_remap.  Bijective on [0, n).
__device__ __forceinline__ int xcd_chunked(int w, int n, int C) {
    const int x = w % kXcds, i = w / kXcds;
    const int full = n / (kXcds * C);
    if (i < full * C) return ((i / C) * kXcds + x) * C + i % C;
    const int base = full * kXcds * C;
    return base + xcd_remap(w - base, n - base);
}

// Tile t of an nm x nn grid in groups of G rows: inside a group the tiles go
// down the rows first, so the tiles that run at the same time cover a few
// rows x a few columns and share the operand panels of both.  Bijective.
__device__ __forceinline__ void grouped_tile(int t, int nm, int nn, int G, int& m, int& n) {
    const int per = G * nn;
    const int g = t / per;
    const int first = g * G;
    const int gs = min(G, nm - first);
    const int local = t - g * per;
    n = local / gs;
    m = first + local % gs;
}

// ------------------------------------------------------------ activations
//
// GeLU in the exact form 0.5 h (1 + erf(h / sqrt 2)).  erf is evaluated with
// the Abramowitz & Stegun 7.1.26 approximation
//   erfc(z) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z),  |error in erf| <= 1.5e-7  (z >= 0),
// with the hardware reciprocal and exp2, at z = |h| / sqrt 2.  The constants
// carry the scale factors: 1/sqrt 2 sits in p, and the exponential is taken
// directly as the normal density phi(h) = exp(-h^2/2) / sqrt(2 pi), so the
// coefficients a_i carry sqrt(2 pi) / 2.  q below is 0.5 erfc(|h|/sqrt 2),
// i.e. Phi(-|h|).
struct ErfcHalf {
    float q;    // Phi(-|h|)
    float phi;  // exp(-h^2 / 2) / sqrt(2 pi)
};

__device__ __forceinline__ ErfcHalf erfc_half(float h) {
    constexpr float kP = 0.3275911f * 0.70710678118654752f;
    constexpr float kS = 0.5f * 2.50662827463100050f;          // sqrt(2 pi) / 2
    constexpr float kE = -0.5f * 1.44269504088896341f;         // -log2(e) / 2
    constexpr float kL = -1.32574806473615971f;                // log2(1 / sqrt(2 pi))
    const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(h), kP, 1.0f));
    float p = fmaf(1.061405429f * kS, t, -1.453152027f * kS);
    p = fmaf(p, t, 1.421413741f * kS);
    p = fmaf(p, t, -0.284496736f * kS);
    p = fmaf(p, t, 0.254829592f * kS);
    const float phi = __builtin_amdgcn_exp2f(fmaf(h, h * kE, kL));
    return {(p * t) * phi, phi};
}

// Phi(h) from q = Phi(-|h|): 1 - q for h > 0, q for h < 0, as |s - q| with
// s = 1 for h > 0 and 0 for h < 0.  s is ldexp(h, 200) clamped to [0, 1], one
// instruction (2^-149 * 2^200 > 1, so every positive float, denormals
// included, gives 1), and the absolute value is a free operand modifier of
// the instructions that use Phi: one instruction instead of a compare, a
// select and 1 - q, with the same values (h = +0 gives q, within rounding
// of 1 - q = 1/2).
__device__ __forceinline__ float phi_cdf(float h, float q) {
    const float s = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(h, 200), 0.0f, 1.0f);
    return fabsf(s - q);
}

__device__ __forceinline__ float gelu_f(float h) {
    const ErfcHalf r = erfc_half(h);
    return h * phi_cdf(h, r.q);
}

// d/dh gelu(h) = Phi(h) + h phi(h)
__device__ __forceinline__ float gelu_grad_f(float h) {
    const ErfcHalf r = erfc_half(h);
    return fmaf(h, r.phi, phi_cdf(h, r.q));
}

// Both at once (one erfc evaluation): what the training forward stores.
__device__ __forceinline__ void gelu_and_grad(float h, float& g, float& gp) {
    const ErfcHalf r = erfc_half(h);
    const float cdf = phi_cdf(h, r.q);
    g = h * cdf;
    gp = fmaf(h, r.phi, cdf);
}

// silu(g) = g / (1 + exp(-g))
__device__ __forceinline__ float silu_f(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}

// silu and its derivative from one exponential: with sigma = 1 / (1 + exp(-g)),
// silu(g) = g sigma and silu'(g) = sigma (1 + g (1 - sigma))
__device__ __forceinline__ void silu_and_grad(float g, float& s, float& sp) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
    s = g * sg;
    sp = sg * fmaf(g, 1.0f - sg, 1.0f);
}


// ------------------------------------------------------------ gate backward
//
// The router-logit gradient of one token, one wave: lane j < k holds dg_j =
// <dy_t, yp_j> and the expert e_j of pick j.  Softmax p of the E logits
// (NV per lane, max-subtracted); dL/dp at the picks (with renorm:
// dg_j / S - (sum_i dg_i p_(e_i)) / S^2, S = sum of the picks' p); scattered
// to the experts' lanes; out[e] = p_e (dL/dp_e - sum_u p_u dL/dp_u).
//
// The logits are loaded apart (load_logits), so a caller can issue that load
// before its other work on the token and hide its latency.
template <int NV>
__device__ __forceinline__ void load_logits(const float* __restrict__ l, int E, float* p) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        p[i] = e < E ? l[e] : -INFINITY;
    }
}

template <int NV>
__device__ __forceinline__ void gate_grad_token_loaded(float* p, int E, int k, int renorm,
                                                       float my_dg, int my_e,
                                                       float* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    // ---- softmax of the logits (max-subtracted)
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) mx = fmaxf(mx, p[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        p[i] = e < E ? expf(p[i] - mx) : 0.0f;
        z += p[i];
    }
    z = wave_sum(z);
    const float rz = 1.0f / z;
#pragma unroll
    for (int i = 0; i < NV; ++i) p[i] *= rz;
    // ---- dL/dp at the picks (lane j: expert e_j)
    float pe = 0.0f;  // p[e_j] on lane j
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float x = __shfl(p[i], my_e & (kWave - 1), kWave);
        if (i == (my_e >> 6)) pe = x;
    }
    float my_dp = my_dg;
    if (renorm) {
        const float S = wave_sum(lane < k ? pe : 0.0f);
        const float D = wave_sum(lane < k ? my_dg * pe : 0.0f);
        my_dp = my_dg / S - D / (S * S);
    }
    // ---- scatter to the experts' lanes, then the softmax Jacobian
    float dp[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) dp[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, kWave);
        const float dj = __shfl(my_dp, j, kWave);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + kWave * i == ej) dp[i] += dj;
    }
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) dot = fmaf(p[i], dp[i], dot);
    dot = wave_sum(dot);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        if (e < E) out[e] = p[i] * (dp[i] - dot);
    }
}

template <int NV>
__device__ __forceinline__ void gate_grad_token(const float* __restrict__ l, int E, int k,
                                                int renorm, float my_dg, int my_e,
                                                float* __restrict__ out) {
    float p[NV];
    load_logits<NV>(l, E, p);
    gate_grad_token_loaded<NV>(p, E, k, renorm, my_dg, my_e, out);
}

}  // namespace bsg
