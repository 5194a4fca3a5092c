/*
 * CPU oracle for the dropless-MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (George Lin's Blog, MegaBlocks/FlexMoE post, section 1.2):
 * the block-sparse formulation is a mathematically equivalent rewrite of the
 * per-expert MLP, so the oracle is the plain definition: a loop over tokens
 * that applies each chosen expert's two-layer MLP densely (first layer
 * x @ W1_e, activation, second layer @ W2_e) and combines the k expert
 * outputs with the gate weights.  Integer outputs (routing, permutation,
 * topology) follow the steps of sections 1.3 and 1.4 of the same post in
 * their order: route, group by expert, pad each group to a multiple of 128,
 * then the hybrid BCSR-COO topology and its transpose index.
 *
 * Arithmetic: every sum is accumulated in fp64 in ascending index order and
 * never reassociated.  Values are rounded to the storage precision at the
 * points where the layer stores an intermediate (A, the saved factors, Yp,
 * y, dYp, dH, dXp, dx, dW); ORC_F64 disables every rounding (used by the finite-difference
 * and library cross-checks).
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes):
 *   - top-k on raw logits, ties to the lower expert id, slots in rank order;
 *   - gate = softmax over all E logits, optionally renormalised over the k
 *     picks;
 *   - stable order inside an expert's bin (ascending assignment id
 *     a = t*k + j), bins in ascending expert id, empty experts get 0 rows,
 *     pad rows are zero;
 *   - exact erf GeLU; SwiGLU = silu(x W1) * (x W3);
 *   - the block-diagonal matrix is the first layer's output [Tp x E*f];
 *   - what the backward keeps of the forward is GeLU'(h) (SwiGLU: silu(h)
 *     and u * silu'(h)), stored (rounded) next to A; the backward multiplies
 *     by it.
 *
 * Parity pins: none of the pages prints a worked numeric example, so every
 * function here is pinned by closed forms, invariants, library routines on
 * special cases, brute force and finite differences in the not-gpu tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F64 0
#define ORC_F32 1
#define ORC_BF16 2

#define ORC_ACT_GELU 0
#define ORC_ACT_SWIGLU 1

#define BLK 128

/* ---------------------------------------------------------------- rounding */

/* Round to bf16 (8 significant bits, fp32 exponent range) with ties to even.
 * The quantum of a value in [2^(e-1), 2^e) is 2^(e-8); below the smallest
 * normal (2^-126) it stays 2^-133. */
static double rd_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    (void)frexp(fabs(v), &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double r = nearbyint(ldexp(fabs(v), -qexp));   /* default mode: ties to even */
    r = ldexp(r, qexp);
    if (r > 3.3895313892515355e38) r = INFINITY; /* beyond the largest bf16 */
    return copysign(r, v);
}

static double rd(double v, int prec) {
    switch (prec) {
    case ORC_F32: return (double)(float)v;
    case ORC_BF16: return rd_bf16(v);
    default: return v;
    }
}

double orc_round(double v, int prec) { return rd(v, prec); }

/* ------------------------------------------------------------ activations */

static double gelu(double h) { return 0.5 * h * (1.0 + erf(h / sqrt(2.0))); }

static double gelu_grad(double h) {
    return 0.5 * (1.0 + erf(h / sqrt(2.0))) + h * exp(-0.5 * h * h) / sqrt(2.0 * M_PI);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* d/dz silu(z) = sigma(z) (1 + z (1 - sigma(z))),  sigma(z) = 1 / (1 + exp(-z)) */
static double silu_grad(double z) {
    const double sg = 1.0 / (1.0 + exp(-z));
    return sg * (1.0 + z * (1.0 - sg));
}

double orc_gelu(double h) { return gelu(h); }
double orc_gelu_grad(double h) { return gelu_grad(h); }
double orc_silu(double z) { return silu(z); }
double orc_silu_grad(double z) { return silu_grad(z); }

/* ---------------------------------------------------------------- threads */

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- routing */

/*
 * Gate network and router (section 1.4 of the MegaBlocks part; the gate and
 * router roles of the FlexMoE section 2.2 component list).  For each token:
 * pick the k experts with the largest logits (ties: lower id first), in rank
 * order; gate = softmax probability over all E experts, renormalised over
 * the k picks when renorm != 0.  Then count tokens per expert, pad each
 * count up to a multiple of bin (128, the block of section 1.3; coarser
 * bins for the block-size study), lay the bins out in ascending expert order
 * (exclusive scan), and give every assignment a = t*k + j the next free row
 * of its expert's bin, visiting assignments in ascending a.
 *
 * row_src (length row_src_len >= Tp) receives the inverse map: the
 * assignment that fills each row, or -1 for a pad row.
 * Returns 0, or -1 on bad arguments.
 */
int orc_route(const float* logits, int64_t T, int E, int k, int renorm, int bin,
              int32_t* expert_idx, float* gate, int32_t* counts, int32_t* bin_offsets,
              int32_t* dest_row, int32_t* row_src, int64_t row_src_len) {
    if (!logits || T < 0 || E < 1 || k < 1 || k > E || bin < 1) return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        /* selection: k passes of "largest not yet taken, lower id on ties" */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int q = 0; q < j; ++q)
                    if (expert_idx[t * k + q] == e) taken = 1;
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            expert_idx[t * k + j] = best;
        }
        /* softmax over all experts in fp64 (max-subtracted) */
        double mx = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += exp((double)l[e] - mx);
        double p[64];
        double* pk = k <= 64 ? p : (double*)malloc(sizeof(double) * k);
        double psum = 0.0;
        for (int j = 0; j < k; ++j) {
            pk[j] = exp((double)l[expert_idx[t * k + j]] - mx) / z;
            psum += pk[j];
        }
        for (int j = 0; j < k; ++j)
            gate[t * k + j] = (float)(renorm ? pk[j] / psum : pk[j]);
        if (pk != p) free(pk);
    }
    /* histogram */
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < T * k; ++a) counts[expert_idx[a]]++;
    /* padded bins, ascending expert id */
    bin_offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int64_t padded = ((int64_t)counts[e] + bin - 1) / bin * bin;
        bin_offsets[e + 1] = (int32_t)(bin_offsets[e] + padded);
    }
    /* stable placement */
    int64_t Tp = bin_offsets[E];
    if (row_src && row_src_len < Tp) return -1;
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (row_src)
        for (int64_t r = 0; r < Tp; ++r) row_src[r] = -1;
    for (int64_t a = 0; a < T * k; ++a) {
        int e = expert_idx[a];
        int32_t row = bin_offsets[e] + fill[e]++;
        dest_row[a] = row;
        if (row_src) row_src[row] = (int32_t)a;
    }
    free(fill);
    return 0;
}

/*
 * Fused permutation + padding (section 1.3 "block size" and section 1.4):
 * row dest_row[a] of xp receives token t = a / k's row of x (times scale[a]
 * when scale is given, rounded to prec); rows that no assignment fills are
 * pad rows and are zero.  xp has Tp rows of d values.
 */
int orc_permute_pad(const float* x, int64_t T, int d, int k, const int32_t* dest_row,
                    const float* scale, int prec, int64_t Tp, double* xp) {
    if (!x || !dest_row || !xp || d < 1 || k < 1) return -1;
    memset(xp, 0, sizeof(double) * (size_t)Tp * (size_t)d);
    for (int64_t a = 0; a < T * k; ++a) {
        int64_t t = a / k;
        int64_t row = dest_row[a];
        if (row < 0 || row >= Tp) return -1;
        for (int i = 0; i < d; ++i) {
            double v = x[t * d + i];
            if (scale) v = (double)scale[a] * v;
            xp[row * d + i] = rd(v, prec);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- topology */

/*
 * Hybrid BCSR-COO topology of the first layer's output, a [Tp x E*f] matrix
 * of 128x128 blocks, and its transpose index (section 1.3, "hybrid BCSR-COO
 * format" and "transpose indices").  Block (r, c) is nonzero when row block r
 * lies in expert e's bin and column block c lies in expert e's f columns.
 *
 * Built the generic way: scan the block grid row by row (BCSR: row_ptr,
 * col_idx; the COO half: row_idx per block), then a stable counting sort of
 * the blocks by column gives col_ptr and trans_idx (BCSR block ids listed in
 * column order, ascending block id inside a column).
 * Row blocks are br rows high (128, the block of section 1.3, or 64 for the
 * block-size study) and 128 columns wide; every bin offset must be a
 * multiple of br.
 * Output sizes: row_ptr [Tp/br + 1], col_ptr [E*F + 1], the others [nnz].
 * Returns nnz, or -1 on bad arguments.
 */
int64_t orc_topology(const int32_t* bin_offsets, int E, int F, int br, int32_t* row_ptr,
                     int32_t* col_idx, int32_t* row_idx, int32_t* col_ptr, int32_t* trans_idx) {
    if (!bin_offsets || E < 1 || F < 1 || br < 1) return -1;
    int64_t Tp = bin_offsets[E];
    for (int e = 0; e <= E; ++e)
        if (bin_offsets[e] % br) return -1;
    int64_t R = Tp / br, C = (int64_t)E * F;
    int64_t nnz = 0;
    for (int64_t r = 0; r < R; ++r) {
        row_ptr[r] = (int32_t)nnz;
        int owner = -1;
        for (int e = 0; e < E; ++e)
            if (r * br >= bin_offsets[e] && r * br < bin_offsets[e + 1]) owner = e;
        for (int64_t c = 0; c < C; ++c) {
            if (c / F == owner) {
                col_idx[nnz] = (int32_t)c;
                row_idx[nnz] = (int32_t)r;
                ++nnz;
            }
        }
    }
    row_ptr[R] = (int32_t)nnz;
    /* transpose: counting sort by column, stable in block id */
    int64_t* cnt = (int64_t*)calloc((size_t)C + 1, sizeof(int64_t));
    for (int64_t b = 0; b < nnz; ++b) cnt[col_idx[b] + 1]++;
    for (int64_t c = 0; c < C; ++c) cnt[c + 1] += cnt[c];
    for (int64_t c = 0; c <= C; ++c) col_ptr[c] = (int32_t)cnt[c];
    for (int64_t b = 0; b < nnz; ++b) trans_idx[cnt[col_idx[b]]++] = (int32_t)b;
    free(cnt);
    return nnz;
}

/*
 * Gate backward: plain calculus on the gate defined above; the top-k
 * selection is piecewise constant and passes no gradient.  For token t with
 * picks e_j and the expert outputs yp_j the forward combined:
 *   dg_j = sum_m dy[t, m] * yp_j[m]
 *   g_j  = p[e_j]   (or p[e_j] / S with S = sum_i p[e_i] when renorm)
 *   dL/dp[e]: the sum of dg_j over the picks j with e_j = e, or with renorm
 *             dg_i / S - (sum_j dg_j p[e_j]) / S^2 at e = e_i, else 0
 *   dlogits[t, e] = p[e] * (dL/dp[e] - sum_u p[u] dL/dp[u])    (softmax)
 * yp holds the T*k rows in assignment order (row a = t*k + j), d values each.
 * Returns 0, or -1 on bad arguments.
 */
int orc_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                       const int32_t* expert_idx, const float* dy, const double* yp, int d,
                       double* dlogits) {
    if (!logits || !expert_idx || !dy || !yp || !dlogits || T < 0 || E < 1 || k < 1 || k > E ||
        d < 1)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * E);
        double* dp = (double*)malloc(sizeof(double) * E);
        double* dg = (double*)malloc(sizeof(double) * k);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float* l = logits + t * E;
            double mx = l[0];
            for (int e = 1; e < E; ++e)
                if (l[e] > mx) mx = l[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)l[e] - mx);
            for (int e = 0; e < E; ++e) p[e] = exp((double)l[e] - mx) / z;
            for (int j = 0; j < k; ++j) {
                const double* y = yp + (t * k + j) * (int64_t)d;
                double s = 0.0;
                for (int m = 0; m < d; ++m) s += (double)dy[t * d + m] * y[m];
                dg[j] = s;
            }
            for (int e = 0; e < E; ++e) dp[e] = 0.0;
            if (renorm) {
                double S = 0.0, D = 0.0;
                for (int j = 0; j < k; ++j) {
                    const int e = expert_idx[t * k + j];
                    if (e < 0 || e >= E) bad = 1;
                    S += p[e];
                }
                for (int j = 0; j < k; ++j) D += dg[j] * p[expert_idx[t * k + j]];
                for (int j = 0; j < k; ++j) dp[expert_idx[t * k + j]] += dg[j] / S - D / (S * S);
            } else {
                for (int j = 0; j < k; ++j) {
                    const int e = expert_idx[t * k + j];
                    if (e < 0 || e >= E) bad = 1;
                    else dp[e] += dg[j];
                }
            }
            double dot = 0.0;
            for (int e = 0; e < E; ++e) dot += p[e] * dp[e];
            for (int e = 0; e < E; ++e) dlogits[t * E + e] = p[e] * (dp[e] - dot);
        }
        free(p);
        free(dp);
        free(dg);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ float layer */

typedef struct {
    int64_t T;
    int d, E, f, k;
    int act;      /* ORC_ACT_GELU or ORC_ACT_SWIGLU */
    int prec;     /* storage precision of A, G, dYp, dH, y, dx, dW */
    int prec_yp;  /* storage precision of Yp and dXp */
    const float* x;   /* [T, d] */
    const float* W1;  /* [d, E*f]: expert e owns columns e*f .. e*f+f-1 */
    const float* W3;  /* [d, E*f] (swiglu only) */
    const float* W2;  /* [E*f, d]: expert e owns rows e*f .. e*f+f-1 */
    const float* dy;  /* [T, d] (backward only) */
    const int32_t* expert_idx; /* [T*k] */
    const float* gate;         /* [T*k] */
} orc_layer;

static int layer_ok(const orc_layer* L) {
    return L && L->x && L->W1 && L->W2 && L->expert_idx && L->gate && L->d > 0 && L->E > 0 &&
           L->f > 0 && L->k > 0 && (L->act != ORC_ACT_SWIGLU || L->W3);
}

/* First layer and activation for one assignment (section 1.2: layer one,
 * then the activation):
 *   h[n] = sum_i x[t,i] W1[i, e*f+n];  SwiGLU also u[n] = sum_i x[t,i] W3[i, e*f+n]
 *   A[n] = rd(gelu(h[n]))  or  rd(silu(h[n]) * u[n])
 * h and u stay unrounded (fp64).  S0 / S1 receive what the backward keeps of
 * the forward, rounded where it is stored (the one rounding point between
 * the passes):
 *   GeLU    S0 = rd(gelu'(h))                       (dH = dA * S0)
 *   SwiGLU  S0 = rd(silu(h)), S1 = rd(u * silu'(h)) (dH_up = dA * S0,
 *                                                    dH_gate = dA * S1) */
static void first_layer(const orc_layer* L, int64_t a, double* h, double* hu, double* S0,
                        double* S1, double* A_out) {
    const int64_t t = a / L->k;
    const int e = L->expert_idx[a];
    const int64_t ldw = (int64_t)L->E * L->f;
    const float* xr = L->x + t * L->d;
    for (int n = 0; n < L->f; ++n) h[n] = 0.0;
    if (hu)
        for (int n = 0; n < L->f; ++n) hu[n] = 0.0;
    /* i outer keeps every h[n] summed in ascending i */
    for (int i = 0; i < L->d; ++i) {
        const double xi = xr[i];
        const float* w = L->W1 + i * ldw + (int64_t)e * L->f;
        for (int n = 0; n < L->f; ++n) h[n] += xi * (double)w[n];
        if (hu) {
            const float* w3 = L->W3 + i * ldw + (int64_t)e * L->f;
            for (int n = 0; n < L->f; ++n) hu[n] += xi * (double)w3[n];
        }
    }
    for (int n = 0; n < L->f; ++n) {
        if (L->act == ORC_ACT_SWIGLU) {
            if (A_out) A_out[n] = rd(silu(h[n]) * hu[n], L->prec);
            if (S0) S0[n] = rd(silu(h[n]), L->prec);
            if (S1) S1[n] = rd(hu[n] * silu_grad(h[n]), L->prec);
        } else {
            if (A_out) A_out[n] = rd(gelu(h[n]), L->prec);
            if (S0) S0[n] = rd(gelu_grad(h[n]), L->prec);
        }
    }
}

/* Second layer for one assignment: Yp[m] = sum_n A[n] W2[e*f+n, m]. */
static void second_layer(const orc_layer* L, int64_t a, const double* A, double* acc, double* Yp) {
    const int e = L->expert_idx[a];
    for (int m = 0; m < L->d; ++m) acc[m] = 0.0;
    for (int n = 0; n < L->f; ++n) {
        const double an = A[n];
        const float* w = L->W2 + ((int64_t)e * L->f + n) * L->d;
        for (int m = 0; m < L->d; ++m) acc[m] += an * (double)w[m];
    }
    for (int m = 0; m < L->d; ++m) Yp[m] = rd(acc[m], L->prec_yp);
}

static double* dalloc(int64_t n) { return (double*)malloc(sizeof(double) * (size_t)n); }

/*
 * Per-assignment forward for the listed assignments, each array [n, f] or
 * [n, d]: S0, S1 the saved factors of first_layer (S1 SwiGLU only; either
 * may be NULL), A the stored activation, Yp the expert output.
 */
int orc_assign_forward(const orc_layer* L, const int64_t* assigns, int64_t n, double* S0,
                       double* S1, double* A, double* Yp) {
    if (!layer_ok(L) || !assigns || !A || !Yp) return -1;
    const int swiglu = L->act == ORC_ACT_SWIGLU;
    int bad = 0;
#pragma omp parallel
    {
        double* h = dalloc(L->f);
        double* hu = swiglu ? dalloc(L->f) : NULL;
        double* acc = dalloc(L->d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t a = assigns[q];
            if (a < 0 || a >= L->T * L->k) {
                bad = 1;
                continue;
            }
            first_layer(L, a, h, hu, S0 ? S0 + q * L->f : NULL,
                        S1 && swiglu ? S1 + q * L->f : NULL, A + q * L->f);
            second_layer(L, a, A + q * L->f, acc, Yp + q * L->d);
        }
        free(h);
        free(hu);
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Layer output for the listed tokens: y[t, m] = sum_j gate[t,j] Yp_{t,j}[m]
 * (j ascending), rounded once.  This is the per-token loop that applies each
 * chosen expert's MLP densely and combines the results with the gates.
 */
int orc_forward_tokens(const orc_layer* L, const int64_t* tokens, int64_t n, double* y) {
    if (!layer_ok(L) || !tokens || !y) return -1;
    int bad = 0;
#pragma omp parallel
    {
        double* h = dalloc(L->f);
        double* hu = L->act == ORC_ACT_SWIGLU ? dalloc(L->f) : NULL;
        double* A = dalloc(L->f);
        double* acc = dalloc(L->d);
        double* yp = dalloc(L->d);
        double* sum = dalloc(L->d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t t = tokens[q];
            if (t < 0 || t >= L->T) {
                bad = 1;
                continue;
            }
            for (int m = 0; m < L->d; ++m) sum[m] = 0.0;
            for (int j = 0; j < L->k; ++j) {
                int64_t a = t * L->k + j;
                first_layer(L, a, h, hu, NULL, NULL, A);
                second_layer(L, a, A, acc, yp);
                const double g = L->gate[a];
                for (int m = 0; m < L->d; ++m) sum[m] += g * yp[m];
            }
            for (int m = 0; m < L->d; ++m) y[q * L->d + m] = rd(sum[m], L->prec);
        }
        free(h);
        free(hu);
        free(A);
        free(acc);
        free(yp);
        free(sum);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- backward */

/* Scratch rows of one backward worker. */
typedef struct {
    double *h, *hu, *S0, *S1, *dYp, *dH, *dHu, *dXp;
} bwd_scratch;

static bwd_scratch bwd_alloc(const orc_layer* L) {
    bwd_scratch w;
    const int sw = L->act == ORC_ACT_SWIGLU;
    w.h = dalloc(L->f);
    w.hu = sw ? dalloc(L->f) : NULL;
    w.S0 = dalloc(L->f);
    w.S1 = sw ? dalloc(L->f) : NULL;
    w.dYp = dalloc(L->d);
    w.dH = dalloc(L->f);
    w.dHu = sw ? dalloc(L->f) : NULL;
    w.dXp = dalloc(L->d);
    return w;
}

static void bwd_free(bwd_scratch* w) {
    free(w->h);
    free(w->hu);
    free(w->S0);
    free(w->S1);
    free(w->dYp);
    free(w->dH);
    free(w->dHu);
    free(w->dXp);
}

/*
 * Backward data path of one assignment (plain calculus on section 1.2's
 * SDD -> activation -> DSD), into w->dYp, w->dH, w->dHu, w->dXp:
 *   dYp[m] = rd(gate * dy[t, m])
 *   da[n]  = sum_m dYp[m] W2[e*f+n, m]
 *   GeLU    dH[n]  = rd(da[n] * S0[n])                 S0 = rd(gelu'(h))
 *           dXp[i] = rd_yp(sum_n dH[n] W1[i, e*f+n])
 *   SwiGLU  dH[n]  = rd(da[n] * S1[n])  gate projection, S1 = rd(u silu'(h))
 *           dHu[n] = rd(da[n] * S0[n])  up projection,   S0 = rd(silu(h))
 *           dXp[i] = rd_yp(sum_n dH[n] W1[i, e*f+n] + sum_n dHu[n] W3[i, e*f+n])
 */
static void assign_backward(const orc_layer* L, int64_t a, bwd_scratch* w) {
    const int64_t t = a / L->k;
    const int e = L->expert_idx[a];
    const int64_t ldw = (int64_t)L->E * L->f;
    const double g = L->gate[a];
    const int sw = L->act == ORC_ACT_SWIGLU;
    first_layer(L, a, w->h, w->hu, w->S0, w->S1, NULL);
    for (int m = 0; m < L->d; ++m) w->dYp[m] = rd(g * (double)L->dy[t * L->d + m], L->prec);
    for (int n = 0; n < L->f; ++n) {
        const float* w2 = L->W2 + ((int64_t)e * L->f + n) * L->d;
        double da = 0.0;
        for (int m = 0; m < L->d; ++m) da += w->dYp[m] * (double)w2[m];
        if (sw) {
            w->dH[n] = rd(da * w->S1[n], L->prec);
            w->dHu[n] = rd(da * w->S0[n], L->prec);
        } else {
            w->dH[n] = rd(da * w->S0[n], L->prec);
        }
    }
    for (int i = 0; i < L->d; ++i) {
        const float* w1 = L->W1 + i * ldw + (int64_t)e * L->f;
        double s = 0.0;
        for (int n = 0; n < L->f; ++n) s += w->dH[n] * (double)w1[n];
        if (sw) {
            const float* w3 = L->W3 + i * ldw + (int64_t)e * L->f;
            double s3 = 0.0;
            for (int n = 0; n < L->f; ++n) s3 += w->dHu[n] * (double)w3[n];
            s += s3;
        }
        w->dXp[i] = rd(s, L->prec_yp);
    }
}

/* Per-assignment backward rows: dYp [n,d], dH [n,f], dHu [n,f] (SwiGLU
 * only; may be NULL), dXp [n,d]. */
int orc_assign_backward(const orc_layer* L, const int64_t* assigns, int64_t n, double* dYp,
                        double* dH, double* dHu, double* dXp) {
    if (!layer_ok(L) || !L->dy || !assigns) return -1;
    const int sw = L->act == ORC_ACT_SWIGLU;
    int bad = 0;
#pragma omp parallel
    {
        bwd_scratch w = bwd_alloc(L);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t a = assigns[q];
            if (a < 0 || a >= L->T * L->k) {
                bad = 1;
                continue;
            }
            assign_backward(L, a, &w);
            if (dYp) memcpy(dYp + q * L->d, w.dYp, sizeof(double) * L->d);
            if (dH) memcpy(dH + q * L->f, w.dH, sizeof(double) * L->f);
            if (dHu && sw) memcpy(dHu + q * L->f, w.dHu, sizeof(double) * L->f);
            if (dXp) memcpy(dXp + q * L->d, w.dXp, sizeof(double) * L->d);
        }
        bwd_free(&w);
    }
    return bad ? -1 : 0;
}

/* Input gradient for the listed tokens: dx[t, i] = rd(sum_j dXp_{t,j}[i]). */
int orc_backward_tokens(const orc_layer* L, const int64_t* tokens, int64_t n, double* dx) {
    if (!layer_ok(L) || !L->dy || !tokens || !dx) return -1;
    int bad = 0;
#pragma omp parallel
    {
        bwd_scratch w = bwd_alloc(L);
        double* sum = dalloc(L->d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t t = tokens[q];
            if (t < 0 || t >= L->T) {
                bad = 1;
                continue;
            }
            for (int i = 0; i < L->d; ++i) sum[i] = 0.0;
            for (int j = 0; j < L->k; ++j) {
                assign_backward(L, t * L->k + j, &w);
                for (int i = 0; i < L->d; ++i) sum[i] += w.dXp[i];
            }
            for (int i = 0; i < L->d; ++i) dx[q * L->d + i] = rd(sum[i], L->prec);
        }
        bwd_free(&w);
        free(sum);
    }
    return bad ? -1 : 0;
}

/* Assignments of expert e in ascending order; returns their count. */
static int64_t expert_assignments(const orc_layer* L, int e, int64_t* out) {
    int64_t c = 0;
    for (int64_t a = 0; a < L->T * L->k; ++a)
        if (L->expert_idx[a] == e) out[c++] = a;
    return c;
}

/* First-layer pre-activations of hidden unit col (= e*f + n) for one
 * assignment: h through W1 and, for SwiGLU, u through W3 (fp64). */
static void hidden_unit(const orc_layer* L, int64_t a, int64_t col, double* h, double* u) {
    const int64_t ldw = (int64_t)L->E * L->f;
    const float* xr = L->x + (a / L->k) * L->d;
    double s = 0.0, s3 = 0.0;
    for (int i = 0; i < L->d; ++i) s += (double)xr[i] * (double)L->W1[i * ldw + col];
    if (L->act == ORC_ACT_SWIGLU)
        for (int i = 0; i < L->d; ++i) s3 += (double)xr[i] * (double)L->W3[i * ldw + col];
    *h = s;
    *u = s3;
}

/*
 * Weight gradient of the second layer (section 1.3 "transpose indices": the
 * weight gradient is the product of the transposed sparse activation with
 * the dense output gradient):
 *   dW2[e*f+n, m] = rd(sum over assignments a of expert e, ascending,
 *                      of A_a[n] * dYp_a[m])
 * for every (rows[p], cols[q]) pair; out is [nr, nc].  Experts with no
 * assignment give exact zeros.
 */
int orc_dW2_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out) {
    if (!layer_ok(L) || !L->dy || !rows || !cols || !out) return -1;
    const int64_t ldw = (int64_t)L->E * L->f;
    int bad = 0;
    for (int64_t s = 0; s < nc; ++s)
        if (cols[s] < 0 || cols[s] >= L->d) bad = 1;
    if (bad) return -1;
    /* Each thread takes a contiguous range of rows, so consecutive rows of
     * one expert share its assignment list and its rounded dYp values
     * (computed once per expert when they fit the cache budget below); the
     * sums themselves are the same, term for term, as per entry. */
#pragma omp parallel
    {
        int64_t* as = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L->T * L->k));
        double* an = dalloc(L->T * L->k);
        double* acc = dalloc(nc);
        double* dyp = NULL;
        int cur_e = -1;
        int64_t c = 0;
#pragma omp for schedule(static)
        for (int64_t p = 0; p < nr; ++p) {
            int64_t row = rows[p];
            if (row < 0 || row >= ldw) {
                bad = 1;
                continue;
            }
            int e = (int)(row / L->f);
            if (e != cur_e) {
                cur_e = e;
                c = expert_assignments(L, e, as);
                free(dyp);
                dyp = c * nc <= ((int64_t)1 << 24) ? dalloc(c * nc) : NULL;
                if (dyp)
                    for (int64_t q = 0; q < c; ++q)
                        for (int64_t s = 0; s < nc; ++s)
                            dyp[q * nc + s] = rd((double)L->gate[as[q]] *
                                                     (double)L->dy[(as[q] / L->k) * L->d + cols[s]],
                                                 L->prec);
            }
            /* A_a[n] for every assignment of the expert */
            for (int64_t q = 0; q < c; ++q) {
                double h, u;
                hidden_unit(L, as[q], row, &h, &u);
                an[q] = rd(L->act == ORC_ACT_SWIGLU ? silu(h) * u : gelu(h), L->prec);
            }
            /* every entry's sum runs over q ascending; the entries of the
             * row are accumulated side by side */
            for (int64_t s = 0; s < nc; ++s) acc[s] = 0.0;
            for (int64_t q = 0; q < c; ++q) {
                const int64_t a = as[q];
                for (int64_t s = 0; s < nc; ++s) {
                    const double g = dyp ? dyp[q * nc + s]
                                         : rd((double)L->gate[a] *
                                                  (double)L->dy[(a / L->k) * L->d + cols[s]],
                                              L->prec);
                    acc[s] += an[q] * g;
                }
            }
            for (int64_t s = 0; s < nc; ++s) out[p * nc + s] = rd(acc[s], L->prec);
        }
        free(acc);
        free(dyp);
        free(as);
        free(an);
    }
    return bad ? -1 : 0;
}

/*
 * Weight gradient of a first-layer projection (proj 0: W1, proj 1: W3,
 * SwiGLU only):
 *   dW[i, e*f+n] = rd(sum over assignments a of expert e, ascending,
 *                     of x[t_a, i] * dH_a[n])
 * with dH the gradient of that projection's pre-activation as in
 * assign_backward, for every (rows[p] = i, cols[q] = e*f+n) pair; out is
 * [nr, nc].
 */
static int input_weight_grad(const orc_layer* L, int proj, const int64_t* rows, int64_t nr,
                             const int64_t* cols, int64_t nc, double* out) {
    if (!layer_ok(L) || !L->dy || !rows || !cols || !out) return -1;
    if (proj == 1 && L->act != ORC_ACT_SWIGLU) return -1;
    const int64_t ldw = (int64_t)L->E * L->f;
    const int sw = L->act == ORC_ACT_SWIGLU;
    int bad = 0;
    for (int64_t p = 0; p < nr; ++p)
        if (rows[p] < 0 || rows[p] >= L->d) bad = 1;
    if (bad) return -1;
    /* Contiguous column ranges per thread: consecutive hidden units of one
     * expert share its assignment list and its rounded dYp rows (kept once
     * per expert when they fit the cache budget below); every sum is the
     * same, term for term, as per entry. */
#pragma omp parallel
    {
        int64_t* as = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L->T * L->k));
        double* dh = dalloc(L->T * L->k);
        double* acc = dalloc(nr);
        double* dyp = NULL;
        int cur_e = -1;
        int64_t c = 0;
#pragma omp for schedule(static)
        for (int64_t s = 0; s < nc; ++s) {
            int64_t col = cols[s];
            if (col < 0 || col >= ldw) {
                bad = 1;
                continue;
            }
            int e = (int)(col / L->f);
            if (e != cur_e) {
                cur_e = e;
                c = expert_assignments(L, e, as);
                free(dyp);
                dyp = c * L->d <= ((int64_t)1 << 24) ? dalloc(c * L->d) : NULL;
                if (dyp)
                    for (int64_t q = 0; q < c; ++q)
                        for (int m = 0; m < L->d; ++m)
                            dyp[q * L->d + m] = rd((double)L->gate[as[q]] *
                                                       (double)L->dy[(as[q] / L->k) * L->d + m],
                                                   L->prec);
            }
            const float* w2 = L->W2 + col * L->d;
            for (int64_t q = 0; q < c; ++q) {
                int64_t a = as[q];
                const int64_t t = a / L->k;
                double h, u;
                hidden_unit(L, a, col, &h, &u);
                double da = 0.0;
                for (int m = 0; m < L->d; ++m) {
                    const double g = dyp ? dyp[q * L->d + m]
                                         : rd((double)L->gate[a] * (double)L->dy[t * L->d + m], L->prec);
                    da += g * (double)w2[m];
                }
                double saved;
                if (!sw) saved = gelu_grad(h);
                else if (proj == 0) saved = u * silu_grad(h);
                else saved = silu(h);
                dh[q] = rd(da * rd(saved, L->prec), L->prec);
            }
            /* every entry's sum runs over q ascending; the entries of the
             * column are accumulated side by side */
            for (int64_t p = 0; p < nr; ++p) acc[p] = 0.0;
            for (int64_t q = 0; q < c; ++q) {
                const float* xr = L->x + (as[q] / L->k) * L->d;
                for (int64_t p = 0; p < nr; ++p) acc[p] += (double)xr[rows[p]] * dh[q];
            }
            for (int64_t p = 0; p < nr; ++p) out[p * nc + s] = rd(acc[p], L->prec);
        }
        free(acc);
        free(dyp);
        free(as);
        free(dh);
    }
    return bad ? -1 : 0;
}

int orc_dW1_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out) {
    return input_weight_grad(L, 0, rows, nr, cols, nc, out);
}

int orc_dW3_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out) {
    return input_weight_grad(L, 1, rows, nr, cols, nc, out);
}

/* ------------------------------------------------------- block products */

/*
 * The three block-sparse products on given operands (section 1.2: SDD, the
 * first layer kept only at the nonzero blocks, then DSD, sparse x dense;
 * section 1.3: DSTD, the transposed sparse operand times a dense one, one
 * block column at a time through the transpose index), for the MoE
 * topology the bins define: blocks are br rows (128, or 64 for the
 * block-size study) by 128 columns, row block r belongs to the expert e
 * whose bin holds row br * r, and expert e owns column blocks
 * e*F .. e*F + F - 1, so nonzero block b = r*F + j sits at (r, e*F + j).  Operands hold the stored
 * values (bf16 widened to fp32); sums run in fp64 over k ascending and are
 * rounded once to prec, after the epilogue.  Block arrays are block-major,
 * [nnz][br][128], a second plane nnz blocks after the first.
 */

/* expert of each row block, from the bins; returns the row-block count */
static int64_t row_owners(const int32_t* bin_offsets, int E, int br, int32_t** owner) {
    const int64_t R = bin_offsets[E] / br;
    int32_t* o = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    for (int64_t r = 0; r < R; ++r) {
        o[r] = -1;
        for (int e = 0; e < E; ++e)
            if (r * br >= bin_offsets[e] && r * br < bin_offsets[e + 1]) o[r] = e;
    }
    *owner = o;
    return R;
}

/* B[k][n] of a dense operand stored as given (trans = 0: b[k*ld + n]) or
 * transposed (trans = 1: b[n*ld + k]) */
static double elem(const float* b, int64_t ld, int trans, int64_t k, int64_t n) {
    return (double)(trans ? b[n * ld + k] : b[k * ld + n]);
}

/*
 * SDD: acc_b[m][n] = sum_k a[br r + m][k] * B[k][128 c + n], k < K, then
 *   epi 0  acc
 *   epi 1  gelu(acc); aux_out (if not NULL) gelu'(acc)
 *   epi 2  silu(acc) * acc2 (acc2 from b2); aux_out (if not NULL) two planes:
 *          silu(acc), acc2 * silu'(acc)
 *   epi 3  acc * aux_in[b]
 *   epi 4  out two planes: acc * aux_in plane 1, acc * aux_in plane 0
 * Returns nnz, or -1 on bad arguments.
 */
int64_t orc_sdd(const float* a, int64_t lda, const float* b, const float* b2, int64_t ldb,
                int trans_b, int K, const int32_t* bin_offsets, int E, int F, int br, int epi,
                const float* aux_in, int prec, double* out, double* aux_out) {
    if (!a || !b || !bin_offsets || !out || K < 1 || E < 1 || F < 1 || br < 1 || epi < 0 ||
        epi > 4)
        return -1;
    if ((epi == 2 && !b2) || ((epi == 3 || epi == 4) && !aux_in)) return -1;
    int32_t* owner;
    const int64_t R = row_owners(bin_offsets, E, br, &owner);
    const int64_t nnz = R * F;
    const int64_t bs = (int64_t)br * BLK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nnz; ++blk) {
        const int64_t r = blk / F, c = (int64_t)owner[r] * F + blk % F;
        double* acc = dalloc(bs);
        double* acc2 = dalloc(bs);
        for (int64_t i = 0; i < bs; ++i) acc[i] = acc2[i] = 0.0;
        for (int64_t m = 0; m < br; ++m) {
            const float* ar = a + (r * br + m) * lda;
            for (int64_t k = 0; k < K; ++k) {
                const double av = ar[k];
                for (int64_t n = 0; n < BLK; ++n) {
                    acc[m * BLK + n] += av * elem(b, ldb, trans_b, k, c * BLK + n);
                    if (epi == 2) acc2[m * BLK + n] += av * elem(b2, ldb, trans_b, k, c * BLK + n);
                }
            }
        }
        for (int64_t i = 0; i < bs; ++i) {
            const double h = acc[i];
            const int64_t o = blk * bs + i;
            switch (epi) {
            case 0: out[o] = rd(h, prec); break;
            case 1:
                out[o] = rd(gelu(h), prec);
                if (aux_out) aux_out[o] = rd(gelu_grad(h), prec);
                break;
            case 2:
                out[o] = rd(silu(h) * acc2[i], prec);
                if (aux_out) {
                    aux_out[o] = rd(silu(h), prec);
                    aux_out[nnz * bs + o] = rd(acc2[i] * silu_grad(h), prec);
                }
                break;
            case 3: out[o] = rd(h * (double)aux_in[o], prec); break;
            default:
                out[o] = rd(h * (double)aux_in[nnz * bs + o], prec);
                out[nnz * bs + o] = rd(h * (double)aux_in[o], prec);
            }
        }
        free(acc);
        free(acc2);
    }
    free(owner);
    return nnz;
}

/*
 * DSD: c[br r + m][n] = sum over the blocks b of row r (ascending), sum_j
 * blocks[b][m][j] * B[128 col(b) + j][n], then the same over blocks2 with
 * B2 from b2 when blocks2 is not NULL; c is [Tp][N] (row-major, N columns).
 * Returns the row count Tp, or -1 on bad arguments.
 */
int64_t orc_dsd(const float* blocks, const float* blocks2, const int32_t* bin_offsets, int E,
                int F, int br, const float* b, const float* b2, int64_t ldb, int trans_b, int N,
                int prec, double* c) {
    if (!blocks || !bin_offsets || !b || !c || E < 1 || F < 1 || br < 1 || N < 1 ||
        (blocks2 && !b2))
        return -1;
    int32_t* owner;
    const int64_t R = row_owners(bin_offsets, E, br, &owner);
    const int64_t bs = (int64_t)br * BLK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < R * br; ++row) {
        const int64_t r = row / br, m = row % br;
        double* acc = dalloc(N);
        for (int n = 0; n < N; ++n) acc[n] = 0.0;
        for (int set = 0; set < (blocks2 ? 2 : 1); ++set) {
            const float* bl = set ? blocks2 : blocks;
            const float* bb = set ? b2 : b;
            for (int j = 0; j < F; ++j) {
                const int64_t blk = r * F + j, col = (int64_t)owner[r] * F + j;
                for (int64_t q = 0; q < BLK; ++q) {
                    const double v = bl[blk * bs + m * BLK + q];
                    for (int n = 0; n < N; ++n) acc[n] += v * elem(bb, ldb, trans_b, col * BLK + q, n);
                }
            }
        }
        for (int n = 0; n < N; ++n) c[row * N + n] = rd(acc[n], prec);
        free(acc);
    }
    free(owner);
    return R * br;
}

/*
 * DSTD: C[128 c + m][n] = sum over the blocks b of block column c, in
 * ascending row (the transpose index's order), sum_j blocks[b][j][m] *
 * dmat[br row(b) + j][n]; C is [E*F*128][N]; a column without blocks (an
 * expert without rows) is zero.  Returns 0, or -1 on bad arguments.
 */
int orc_dstd(const float* blocks, const int32_t* bin_offsets, int E, int F, int br,
             const float* dmat, int64_t ldd, int N, int prec, double* C) {
    if (!blocks || !bin_offsets || !dmat || !C || E < 1 || F < 1 || br < 1 || N < 1) return -1;
    const int64_t bs = (int64_t)br * BLK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t out_row = 0; out_row < (int64_t)E * F * BLK; ++out_row) {
        const int64_t c = out_row / BLK, m = out_row % BLK;
        const int e = (int)(c / F), j = (int)(c % F);
        double* acc = dalloc(N);
        for (int n = 0; n < N; ++n) acc[n] = 0.0;
        for (int64_t r = bin_offsets[e] / br; r < bin_offsets[e + 1] / br; ++r) {
            const int64_t blk = r * F + j;
            for (int64_t q = 0; q < br; ++q) {
                const double v = blocks[blk * bs + q * BLK + m];
                const float* dr = dmat + (r * br + q) * ldd;
                for (int n = 0; n < N; ++n) acc[n] += v * (double)dr[n];
            }
        }
        for (int n = 0; n < N; ++n) C[out_row * N + n] = rd(acc[n], prec);
        free(acc);
    }
    return 0;
}
