// Driver for the sanitizer build: the C ABI's argument validation (api.cpp,
// launchers replaced by host stand-ins) and every entry point of the CPU
// oracle, run under AddressSanitizer and UndefinedBehaviorSanitizer.  Exits
// 0 when every expectation holds; a sanitizer report aborts the run.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../block_sparse_gemm_amd/csrc/kernels.hpp"
#include "../../include/bsg.h"

extern int g_launches;
extern bsg::TopoJob g_route_topo;
extern bsg::PermJob g_route_perm;
extern bsg::GemmParams g_dsd;

// ---- the oracle's C entry points (oracle/oracle.c)
extern "C" {
typedef struct {
    int64_t T;
    int d, E, f, k;
    int act, prec, prec_yp;
    const float *x, *W1, *W3, *W2, *dy;
    const int32_t* expert_idx;
    const float* gate;
} orc_layer;
double orc_round(double v, int prec);
double orc_gelu(double h);
double orc_gelu_grad(double h);
double orc_silu(double z);
double orc_silu_grad(double z);
void orc_set_threads(int n);
int orc_route(const float* logits, int64_t T, int E, int k, int renorm, int bin,
              int32_t* expert_idx, float* gate, int32_t* counts, int32_t* bin_offsets,
              int32_t* dest_row, int32_t* row_src, int64_t row_src_len);
int orc_permute_pad(const float* x, int64_t T, int d, int k, const int32_t* dest_row,
                    const float* scale, int prec, int64_t Tp, double* xp);
int64_t orc_topology(const int32_t* bin_offsets, int E, int F, int br, int32_t* row_ptr,
                     int32_t* col_idx, int32_t* row_idx, int32_t* col_ptr, int32_t* trans_idx);
int orc_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                       const int32_t* expert_idx, const float* dy, const double* yp, int d,
                       double* dlogits);
int orc_assign_forward(const orc_layer* L, const int64_t* assigns, int64_t n, double* S0,
                       double* S1, double* A, double* Yp);
int orc_forward_tokens(const orc_layer* L, const int64_t* tokens, int64_t n, double* y);
int orc_assign_backward(const orc_layer* L, const int64_t* assigns, int64_t n, double* dYp,
                        double* dH, double* dHu, double* dXp);
int orc_backward_tokens(const orc_layer* L, const int64_t* tokens, int64_t n, double* dx);
int orc_dW2_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out);
int orc_dW1_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out);
int orc_dW3_block(const orc_layer* L, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* out);
}

static int g_fail = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
                    __LINE__, #cond);                                        \
            g_fail = 1;                                                      \
        }                                                                    \
    } while (0)

// fake, aligned, never dereferenced device pointers
static void* const P = (void*)0x10000;
static void* const MIS = (void*)0x10004;

static bsg_topology fake_topo(int E, int f, int64_t Tp) {
    bsg_topology t;
    t.row_ptr = (int32_t*)0x10000;
    t.col_idx = (int32_t*)0x20000;
    t.row_idx = (int32_t*)0x30000;
    t.col_ptr = (int32_t*)0x40000;
    t.trans_idx = (int32_t*)0x50000;
    t.row_tiles = (int32_t*)0x70000;
    t.expert_order = (int32_t*)0x80000;
    t.meta = (int32_t*)0x60000;
    t.E = E;
    t.F = f / 128;
    t.block_rows = 128;
    t.Tp_max = Tp;
    return t;
}

static void abi_checks() {
    const float* fl = (const float*)P;
    int32_t* ip = (int32_t*)P;
    float* fp = (float*)P;
    // size queries at ordinary and extreme sizes
    EXPECT(bsg_max_padded_rows(32768, 1, 64, 128) == (32768 + 127 * 64) / 128 * 128);
    EXPECT(bsg_max_padded_rows(INT64_MAX, 32, 1024, 128) == -1);
    EXPECT(bsg_max_padded_rows(INT64_MAX / 2, 2, 8, 256) == -1);
    EXPECT(bsg_max_padded_rows(-5, 1, 1, 128) == -1);
    EXPECT(bsg_route_workspace_bytes(INT64_MAX, 32, 1024) == 0);
    EXPECT(bsg_route_workspace_bytes(65536, 2, 64) == 1024 * 64 * 4);
    bsg_topo_sizes ts;
    EXPECT(bsg_topology_sizes(139136, 64, 4096, 128, &ts) == BSG_OK && ts.nnz_max == 1087 * 32);
    EXPECT(bsg_topology_sizes(139136, 64, 4096, 64, &ts) == BSG_OK && ts.nnz_max == 2174 * 32);
    EXPECT(bsg_topology_sizes(INT64_MAX / 128 * 128, 1024, 128 << 20, 64, &ts) == BSG_EINVAL);
    EXPECT(bsg_topology_sizes(1280, 4, 200, 128, &ts) == BSG_EINVAL);
    EXPECT(bsg_topology_sizes(1280, 4, 256, 100, &ts) == BSG_EINVAL);
    EXPECT(bsg_topology_sizes(1280, 4, 256, 128, nullptr) == BSG_EINVAL);

    // route and its allocation-free twin
    const int before = g_launches;
    EXPECT(bsg_route(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) == BSG_OK);
    EXPECT(bsg_route_noalloc(fl, 100, 8, 2, 0, 256, ip, fp, ip, ip, ip, nullptr) == BSG_OK);
    EXPECT(g_launches == before + 2);
    EXPECT(bsg_route(fl, INT64_MAX, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) ==
           BSG_EINVAL);
    EXPECT(bsg_route_noalloc(fl, INT64_MAX / 3, 8, 4, 0, 128, ip, fp, ip, ip, ip, nullptr) ==
           BSG_EINVAL);
    EXPECT(bsg_route(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 4, nullptr) == BSG_EINVAL);
    EXPECT(strlen(bsg_last_error()) > 0);
    EXPECT(bsg_route_noalloc(fl, 64 * 1025, 1024, 1, 0, 128, ip, fp, ip, ip, ip, nullptr) ==
           BSG_EUNSUPPORTED);
    EXPECT(bsg_route(nullptr, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) ==
           BSG_EINVAL);
    EXPECT(bsg_route(fl, 100, 8, 2, 0, 64, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) == BSG_OK);
    EXPECT(bsg_route(fl, 100, 8, 2, 0, 32, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) ==
           BSG_EINVAL);

    // permute_pad, the gate backward, combine
    const int64_t Tp = bsg_max_padded_rows(100, 2, 8, 128);
    EXPECT(bsg_permute_pad(P, BSG_BF16, 100, 128, 2, ip, nullptr, ip, ip, 8, 128, Tp, ip, P,
                           nullptr) == BSG_OK);
    EXPECT(bsg_permute_pad(P, BSG_BF16, INT64_MAX, 128, 2, ip, nullptr, ip, ip, 8, 128, Tp, ip,
                           P, nullptr) == BSG_EINVAL);
    EXPECT(bsg_permute_pad(P, BSG_BF16, 100, 128, 2, ip, nullptr, ip, ip, 8, 128, Tp - 128, ip,
                           P, nullptr) == BSG_EINVAL);
    EXPECT(bsg_permute_pad_gate_backward(P, BSG_BF16, 100, 128, 2, ip, fp, ip, ip, 8, 128, Tp,
                                         ip, P, fl, 0, ip, P, BSG_BF16, 128, fp,
                                         nullptr) == BSG_OK);
    EXPECT(bsg_permute_pad_gate_backward(P, BSG_BF16, 100, 128, 2, ip, fp, ip, ip, 8, 128, Tp,
                                         ip, P, fl, 0, ip, MIS, BSG_BF16, 128, fp,
                                         nullptr) == BSG_EINVAL);
    EXPECT(bsg_route_backward(fl, 100, 8, 2, 0, ip, ip, P, BSG_BF16, 128, P, BSG_BF16, 128, fp,
                              nullptr) == BSG_OK);
    EXPECT(bsg_route_backward(fl, INT64_MAX, 8, 2, 0, ip, ip, P, BSG_BF16, 128, P, BSG_BF16, 128,
                              fp, nullptr) == BSG_EINVAL);
    EXPECT(bsg_unpermute_combine(P, BSG_BF16, 128, ip, nullptr, 10, 2, 128, P, BSG_BF16,
                                 nullptr) == BSG_OK);
    EXPECT(bsg_unpermute_combine(P, BSG_BF16, 128, ip, nullptr, INT64_MAX, 2, 128, P, BSG_BF16,
                                 nullptr) == BSG_EINVAL);

    // topology and products
    bsg_topology t = fake_topo(4, 256, 1024);
    EXPECT(bsg_build_topology(ip, 4, 256, 1024, &t, nullptr) == BSG_OK);
    t.block_rows = 64;
    EXPECT(bsg_build_topology(ip, 4, 256, 1024, &t, nullptr) == BSG_OK);
    EXPECT(bsg_sdd(P, 256, P, nullptr, 1024, 0, 256, &t, BSG_EPI_GELU, nullptr, P, P, BSG_BF16,
                   nullptr) == BSG_OK);
    t.block_rows = 32;
    EXPECT(bsg_build_topology(ip, 4, 256, 1024, &t, nullptr) == BSG_EINVAL);
    t.block_rows = 128;
    EXPECT(bsg_build_topology(ip, 5, 256, 1024, &t, nullptr) == BSG_EINVAL);
    bsg_topology big = fake_topo(1024, 128 * 32768, INT64_MAX / 128 * 128);
    EXPECT(bsg_build_topology(ip, 1024, 128 * 32768, big.Tp_max, &big, nullptr) == BSG_EINVAL);
    // route + topology in one call: the routing launch carries the topology
    {
        bsg_topology rt = fake_topo(8, 256, bsg_max_padded_rows(100, 2, 8, 128));
        const int n0 = g_launches;
        EXPECT(bsg_route_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, 256,
                                  rt.Tp_max, &rt, nullptr) == BSG_OK);
        EXPECT(g_launches == n0 + 1 && g_route_topo.on == 1 && g_route_topo.F == 2 &&
               g_route_topo.br == 128 && g_route_topo.o.meta == rt.meta &&
               g_route_topo.row_blocks_max == rt.Tp_max / 128);
        EXPECT(bsg_route(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, nullptr) ==
                   BSG_OK &&
               g_route_topo.on == 0);
        EXPECT(bsg_route_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, 384,
                                  rt.Tp_max, &rt, nullptr) == BSG_EINVAL);
        EXPECT(bsg_route_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 4, 256,
                                  rt.Tp_max, &rt, nullptr) == BSG_EINVAL);
        EXPECT(bsg_route_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, 256,
                                  rt.Tp_max, nullptr, nullptr) == BSG_EINVAL);
        EXPECT(g_launches == n0 + 2);
        // ... and with the permutation as well (topology optional)
        const int n1 = g_launches;
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, P,
                                          BSG_BF16, 256, rt.Tp_max, ip, P, 256, &rt,
                                          nullptr) == BSG_OK);
        EXPECT(g_launches == n1 + 1 && g_route_topo.on == 1 && g_route_perm.on == 1 &&
               g_route_perm.chunks == 32 && g_route_perm.Tp_max == rt.Tp_max);
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, P,
                                          BSG_F32, 128, rt.Tp_max, ip, P, 0, nullptr,
                                          nullptr) == BSG_OK);
        EXPECT(g_route_topo.on == 0 && g_route_perm.on == 1 && g_route_perm.chunks == 32);
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20,
                                          MIS, BSG_BF16, 256, rt.Tp_max, ip, P, 256, &rt,
                                          nullptr) == BSG_EINVAL);
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, P,
                                          BSG_BF16, 100, rt.Tp_max, ip, P, 256, &rt,
                                          nullptr) == BSG_EINVAL);
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, P,
                                          BSG_BF16, 256, rt.Tp_max - 128, ip, P, 256, nullptr,
                                          nullptr) == BSG_EINVAL);
        EXPECT(bsg_route_permute_topology(fl, 100, 8, 2, 0, 128, ip, fp, ip, ip, ip, P, 1 << 20, P,
                                          BSG_BF16, 256, rt.Tp_max, ip, P, 384, &rt,
                                          nullptr) == BSG_EINVAL);
        EXPECT(g_launches == n1 + 2);
    }
    EXPECT(bsg_sdd(P, 256, P, nullptr, 1024, 0, 256, &t, BSG_EPI_GELU, nullptr, P, P, BSG_BF16,
                   nullptr) == BSG_OK);
    EXPECT(bsg_sdd(P, 256, P, P, 1024, 0, 256, &t, BSG_EPI_SILU_MUL, nullptr, P, P, BSG_BF16,
                   nullptr) == BSG_OK);
    EXPECT(bsg_sdd(P, 256, P, nullptr, 256, 1, 256, &t, BSG_EPI_GELU_BWD, P, P, nullptr,
                   BSG_BF16, nullptr) == BSG_OK);
    EXPECT(bsg_sdd(P, INT64_MAX, P, nullptr, 1024, 0, 256, &t, BSG_EPI_GELU, nullptr, P, P,
                   BSG_BF16, nullptr) == BSG_EINVAL);
    EXPECT(bsg_sdd(P, 16909320, P, nullptr, 1024, 0, 256, &t, BSG_EPI_GELU, nullptr, P, P,
                   BSG_BF16, nullptr) == BSG_EUNSUPPORTED);
    EXPECT(bsg_dsd(P, nullptr, &t, P, nullptr, 256, 0, 256, P, 256, BSG_BF16, BSG_BF16,
                   nullptr, 0, nullptr) == BSG_OK);
    EXPECT(bsg_dsd(P, P, &t, P, P, 1024, 1, 256, P, 256, BSG_F32, BSG_BF16, nullptr, 0,
                   nullptr) == BSG_OK);
    EXPECT(bsg_dsd(P, nullptr, &t, P, nullptr, INT64_MAX, 0, 256, P, 256, BSG_BF16, BSG_BF16,
                   nullptr, 0, nullptr) == BSG_EINVAL);
    // the workspace: ignored for short tiles (F = 4 K-blocks a row here),
    // rejected when misaligned or under two shares
    EXPECT(bsg_dsd(P, nullptr, &t, P, nullptr, 256, 0, 256, P, 256, BSG_BF16, BSG_BF16, P,
                   1 << 20, nullptr) == BSG_OK &&
           g_dsd.ws == nullptr);
    EXPECT(bsg_dsd(P, nullptr, &t, P, nullptr, 256, 0, 256, P, 256, BSG_BF16, BSG_BF16, MIS,
                   1 << 20, nullptr) == BSG_EINVAL);
    EXPECT(bsg_dsd(P, nullptr, &t, P, nullptr, 256, 0, 256, P, 256, BSG_BF16, BSG_BF16, P,
                   BSG_DSD_SHARE_BYTES, nullptr) == BSG_EINVAL);
    {
        int64_t wsb = 0;
        EXPECT(bsg_dsd_workspace_bytes(nullptr, &wsb) == BSG_OK &&
               wsb == 256 * (int64_t)BSG_DSD_SHARE_BYTES);
        EXPECT(bsg_dsd_workspace_bytes(nullptr, nullptr) == BSG_EINVAL);
        // long tiles (f = 4096: 32 K-blocks) take the split
        bsg_topology lt = fake_topo(4, 4096, 1024);
        EXPECT(bsg_dsd(P, nullptr, &lt, P, nullptr, 256, 0, 256, P, 256, BSG_BF16, BSG_BF16, P,
                       3 * (size_t)BSG_DSD_SHARE_BYTES, nullptr) == BSG_OK &&
               g_dsd.ws == (float*)P && g_dsd.ws_units == 3 && g_dsd.ncu == 256);
    }
    EXPECT(bsg_dsd_combine_top1(P, &t, P, 256, 0, 256, nullptr, 0, ip, fp, P, 256, BSG_BF16,
                                nullptr) == BSG_OK);
    EXPECT(bsg_dstd(P, &t, P, 256, 256, P, 1024, 1, BSG_BF16, nullptr) == BSG_OK);
    EXPECT(bsg_dstd(P, &t, P, INT64_MAX, 256, P, 1024, 1, BSG_BF16, nullptr) == BSG_EINVAL);
    EXPECT(bsg_stream_copy(P, (void*)0x100000, 4096, nullptr) == BSG_OK);
    EXPECT(bsg_stream_copy(P, (void*)0x10010, 4096, nullptr) == BSG_EINVAL);
    EXPECT(bsg_stream_copy(P, (void*)0x100000, SIZE_MAX - 15, nullptr) == BSG_EINVAL);
    EXPECT(strcmp(bsg_status_string(BSG_EHIP), "HIP runtime error") == 0);
    EXPECT(strcmp(bsg_status_string((bsg_status)7), "unknown status") == 0);
}

static void oracle_checks() {
    orc_set_threads(2);
    const int64_t T = 70;
    const int d = 16, E = 3, f = 12, k = 2;
    std::vector<float> logits(T * E), x(T * d), W1(d * E * f), W3(d * E * f), W2(E * f * d),
        dy(T * d);
    uint32_t s = 12345;
    auto rnd = [&]() {
        s = s * 1664525u + 1013904223u;
        return ((s >> 8) & 0xffff) / 32768.0f - 1.0f;
    };
    for (auto* v : {&logits, &x, &W1, &W3, &W2, &dy})
        for (float& a : *v) a = rnd();
    std::vector<int32_t> ei(T * k), counts(E), bo(E + 1), dest(T * k);
    std::vector<float> gate(T * k);
    const int64_t cap = (T * k + 127 * E) / 128 * 128;
    std::vector<int32_t> row_src(cap);
    EXPECT(orc_route(logits.data(), T, E, k, 1, 128, ei.data(), gate.data(), counts.data(),
                     bo.data(), dest.data(), row_src.data(), cap) == 0);
    const int64_t Tp = bo[E];
    std::vector<double> xp(Tp * d);
    std::vector<float> scale(T * k, 0.75f);
    EXPECT(orc_permute_pad(x.data(), T, d, k, dest.data(), scale.data(), 2, Tp, xp.data()) == 0);
    const int F = 2;
    std::vector<int32_t> rp(Tp / 128 + 1), ci(Tp / 128 * F), ri(Tp / 128 * F), cp(E * F + 1),
        tr(Tp / 128 * F);
    EXPECT(orc_topology(bo.data(), E, F, 128, rp.data(), ci.data(), ri.data(), cp.data(),
                        tr.data()) == Tp / 128 * F);
    for (int act = 0; act < 2; ++act)
        for (int prec = 0; prec < 3; ++prec) {
            orc_layer L = {T, d, E, f, k, act, prec, prec, x.data(), W1.data(), W3.data(),
                           W2.data(), dy.data(), ei.data(), gate.data()};
            std::vector<int64_t> as(T * k), toks(T), rows(E * f), cols(d);
            for (int64_t i = 0; i < T * k; ++i) as[i] = i;
            for (int64_t i = 0; i < T; ++i) toks[i] = i;
            for (int64_t i = 0; i < E * f; ++i) rows[i] = i;
            for (int64_t i = 0; i < d; ++i) cols[i] = i;
            std::vector<double> S0(T * k * f), S1(T * k * f), A(T * k * f), Yp(T * k * d),
                y(T * d), dYp(T * k * d), dH(T * k * f), dHu(T * k * f), dXp(T * k * d),
                dx(T * d), dW2(E * f * d), dW1(d * E * f), dW3(d * E * f), dl(T * E);
            EXPECT(orc_assign_forward(&L, as.data(), T * k, S0.data(), S1.data(), A.data(),
                                      Yp.data()) == 0);
            EXPECT(orc_forward_tokens(&L, toks.data(), T, y.data()) == 0);
            EXPECT(orc_assign_backward(&L, as.data(), T * k, dYp.data(), dH.data(), dHu.data(),
                                       dXp.data()) == 0);
            EXPECT(orc_backward_tokens(&L, toks.data(), T, dx.data()) == 0);
            EXPECT(orc_dW2_block(&L, rows.data(), E * f, cols.data(), d, dW2.data()) == 0);
            EXPECT(orc_dW1_block(&L, cols.data(), d, rows.data(), E * f, dW1.data()) == 0);
            EXPECT(orc_dW3_block(&L, cols.data(), d, rows.data(), E * f, dW3.data()) ==
                   (act == 1 ? 0 : -1));
            EXPECT(orc_route_backward(logits.data(), T, E, k, 1, ei.data(), dy.data(), Yp.data(),
                                      d, dl.data()) == 0);
            // out-of-range requests are refused, not read
            const int64_t bad[1] = {T * k};
            EXPECT(orc_assign_forward(&L, bad, 1, S0.data(), S1.data(), A.data(), Yp.data()) ==
                   -1);
            const int64_t badrow[1] = {E * f};
            EXPECT(orc_dW2_block(&L, badrow, 1, cols.data(), d, dW2.data()) == -1);
            for (double v : y) EXPECT(isfinite(v));
            for (double v : dW1) EXPECT(isfinite(v));
        }
    EXPECT(orc_round(1.0 + 1.0 / 512, 2) == 1.0);
    EXPECT(orc_gelu(0.0) == 0.0 && orc_gelu_grad(0.0) == 0.5);
    EXPECT(orc_silu(0.0) == 0.0 && orc_silu_grad(0.0) == 0.5);
}

int main() {
    abi_checks();
    oracle_checks();
    if (g_fail) return 1;
    printf("sanitized checks passed\n");
    return 0;
}
