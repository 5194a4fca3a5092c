// C ABI of the block-sparse expert layer: argument validation, size
// queries and kernel launches.  Every check runs before any HIP call, so
// argument errors are reported without touching a GPU.
#include "../../include/bsg.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "kernels.hpp"

static_assert(bsg::kRouteScratchBytes == BSG_ROUTE_SCRATCH_BYTES, "one scratch size");
static_assert(bsg::kSplitShareBytes == BSG_DSD_SHARE_BYTES, "one share size");

namespace {

thread_local char g_err[512] = "";

bsg_status fail(bsg_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bsg_status ok() {
    g_err[0] = '\0';
    return BSG_OK;
}

bsg_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(BSG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Bounds checked before any size is multiplied, so that validation itself
// never overflows: tokens and block rows fit int32 ids, leading dimensions
// and widths stay far below the point where a byte count would wrap.
constexpr int64_t kMaxLd = int64_t(1) << 40;
constexpr int kMaxWidth = 1 << 24;

int elt_bytes(int dtype) { return dtype == BSG_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == BSG_F32 || dtype == BSG_BF16; }

#define REQUIRE(cond, ...)                                 \
    do {                                                   \
        if (!(cond)) return fail(BSG_EINVAL, __VA_ARGS__); \
    } while (0)

// A device array read or written with 16-byte vectors.
#define REQUIRE_VEC_PTR(p) REQUIRE((p) != nullptr && aligned((p), 16), #p " must be a non-null 16-byte aligned device pointer")
// A device array of 4-byte elements.
#define REQUIRE_PTR(p) REQUIRE((p) != nullptr && aligned((p), 4), #p " must be a non-null 4-byte aligned device pointer")

bsg_status check_topology(const bsg_topology* t) {
    REQUIRE(t != nullptr, "topo is NULL");
    REQUIRE(t->E >= 1 && t->E <= BSG_MAX_EXPERTS, "topo->E out of range");
    REQUIRE(t->F >= 1, "topo->F must be positive");
    REQUIRE(t->block_rows == 128 || t->block_rows == 64, "topo->block_rows must be 128 or 64");
    REQUIRE(t->Tp_max >= t->block_rows && t->Tp_max % t->block_rows == 0,
            "topo->Tp_max must be a positive multiple of topo->block_rows");
    // row_tiles entries keep the first block row in 23 bits
    REQUIRE(t->Tp_max / t->block_rows < (int64_t(1) << 23), "too many block rows for row tiles");
    REQUIRE(t->Tp_max / t->block_rows <= INT32_MAX &&
                (t->Tp_max / t->block_rows) * (int64_t)t->F < INT32_MAX &&
                (int64_t)t->E * t->F < INT32_MAX,
            "too many blocks for int32 ids");
    REQUIRE_PTR(t->row_ptr);
    REQUIRE_PTR(t->col_idx);
    REQUIRE_PTR(t->row_idx);
    REQUIRE_PTR(t->col_ptr);
    REQUIRE_PTR(t->trans_idx);
    REQUIRE_PTR(t->row_tiles);
    REQUIRE_PTR(t->expert_order);
    REQUIRE_PTR(t->meta);
    return BSG_OK;
}

// The products address an operand panel's rows through 32-bit per-lane
// byte offsets from the panel's origin (the largest: row 127 of a panel
// whose rows are contiguous along K, or K-row 31 (bf16) / 15 (fp32) of a
// panel whose rows are contiguous along M or N).  A leading dimension whose
// largest offset does not fit is refused rather than wrapped.
bool panel_ld_fits(int64_t ld, int es, bool k_contiguous) {
    const int64_t last_row = k_contiguous ? 127 : (es == 2 ? 31 : 15);
    const int64_t row_bytes = k_contiguous ? 64 : 256 * (es == 2 ? 1 : 2);
    return last_row * ld * es + row_bytes <= (int64_t)UINT32_MAX;
}

#define REQUIRE_PANEL_LD(ld, es, kc)                                                       \
    do {                                                                                   \
        if (!panel_ld_fits((ld), (es), (kc)))                                              \
            return fail(BSG_EUNSUPPORTED, #ld " = %lld is too large for the products' "    \
                        "32-bit panel offsets", (long long)(ld));                          \
    } while (0)

// Product tiles of 256 rows: each expert's R_e block rows of br rows make
// ceil(R_e / Q) tiles (Q = 256 / br), so their sum is at most
// (R + (Q - 1) * ne) / Q over the ne <= min(E, R) non-empty experts.
int64_t row_tiles_max(int64_t row_blocks_max, int E, int br) {
    const int64_t q = 256 / br;
    const int64_t ne = E < row_blocks_max ? E : row_blocks_max;
    return (row_blocks_max + (q - 1) * (ne + 1)) / q;
}

}  // namespace

extern "C" {

const char* bsg_status_string(bsg_status s) {
    switch (s) {
    case BSG_OK: return "ok";
    case BSG_EINVAL: return "invalid argument";
    case BSG_EUNSUPPORTED: return "unsupported combination";
    case BSG_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char* bsg_last_error(void) { return g_err; }

int64_t bsg_max_padded_rows(int64_t T, int k, int E, int bin_rows) {
    if (T < 1 || T > INT32_MAX || k < 1 || E < 1 || k > E ||
        (bin_rows != 64 && bin_rows != 128 && bin_rows != 256))
        return -1;
    const int64_t A = T * k;
    const int64_t ne = A < E ? A : E;
    return (A + (bin_rows - 1) * ne) / bin_rows * bin_rows;
}

bsg_status bsg_topology_sizes(int64_t Tp_max, int E, int f, int block_rows,
                              bsg_topo_sizes* out) {
    REQUIRE(out != nullptr, "out is NULL");
    REQUIRE(block_rows == 128 || block_rows == 64, "block_rows must be 128 or 64");
    REQUIRE(Tp_max >= block_rows && Tp_max % block_rows == 0,
            "Tp_max must be a positive multiple of block_rows");
    REQUIRE(E >= 1 && E <= BSG_MAX_EXPERTS, "E must be in [1, %d]", BSG_MAX_EXPERTS);
    REQUIRE(f >= BSG_BLOCK && f % BSG_BLOCK == 0, "f must be a positive multiple of 128");
    REQUIRE(Tp_max / block_rows <= INT32_MAX, "too many block rows for int32 ids");
    const int64_t F = f / BSG_BLOCK;
    out->row_blocks_max = Tp_max / block_rows;
    out->nnz_max = out->row_blocks_max * F;
    out->n_cols = (int64_t)E * F;
    out->row_tiles_max = row_tiles_max(out->row_blocks_max, E, block_rows);
    REQUIRE(out->nnz_max < INT32_MAX && out->n_cols < INT32_MAX, "too many blocks for int32 ids");
    return ok();
}

size_t bsg_route_workspace_bytes(int64_t T, int k, int E) {
    if (T < 1 || T > INT32_MAX || k < 1 || E < 1 || k > E) return 0;
    const int64_t nchunks = (T + bsg::kRouteChunk - 1) / bsg::kRouteChunk;
    return (size_t)(nchunks * E * (int64_t)sizeof(int32_t));
}

// The bin granularity: 128 (the block), or 64 or 256 for the block-size
// study (bins of 64 rows go with a topology of 64-row blocks).
static bsg_status check_bin(int bin_rows) {
    REQUIRE(bin_rows == 64 || bin_rows == 128 || bin_rows == 256,
            "bin_rows must be 64, 128 or 256");
    return BSG_OK;
}

static bsg_status check_route(const float* logits, int64_t T, int E, int k, int bin_rows,
                              int32_t* expert_idx, float* gate, int32_t* dest_row,
                              int32_t* counts, int32_t* bin_offsets) {
    const bsg_status bs = check_bin(bin_rows);
    if (bs != BSG_OK) return bs;
    REQUIRE(T >= 1, "T must be positive");
    REQUIRE(E >= 1 && E <= BSG_MAX_EXPERTS, "E must be in [1, %d]", BSG_MAX_EXPERTS);
    REQUIRE(k >= 1 && k <= E, "k must be in [1, E]");
    if (k > BSG_MAX_TOPK) return fail(BSG_EUNSUPPORTED, "k > %d is not implemented", BSG_MAX_TOPK);
    REQUIRE(T <= INT32_MAX && T * k < INT32_MAX, "T*k must fit int32 assignment ids");
    REQUIRE(bsg_max_padded_rows(T, k, E, bin_rows) < INT32_MAX, "padded rows must fit int32");
    REQUIRE_PTR(logits);
    REQUIRE_PTR(expert_idx);
    REQUIRE_PTR(gate);
    REQUIRE_PTR(dest_row);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(bin_offsets);
    return BSG_OK;
}

bsg_status bsg_route(const float* logits, int64_t T, int E, int k, int renorm, int bin_rows,
                     int32_t* expert_idx, float* gate, int32_t* dest_row, int32_t* counts,
                     int32_t* bin_offsets, void* workspace, size_t workspace_bytes,
                     bsg_stream_t stream) {
    const bsg_status s =
        check_route(logits, T, E, k, bin_rows, expert_idx, gate, dest_row, counts, bin_offsets);
    if (s != BSG_OK) return s;
    REQUIRE_PTR(workspace);
    REQUIRE(workspace_bytes >= bsg_route_workspace_bytes(T, k, E), "workspace too small (%zu < %zu)",
            workspace_bytes, bsg_route_workspace_bytes(T, k, E));
    return hip_status(bsg::launch_route(logits, T, E, k, renorm, bin_rows, expert_idx, gate, dest_row,
                                        counts, bin_offsets, (int32_t*)workspace, bsg::TopoJob{},
                                        bsg::PermJob{}, (hipStream_t)stream),
                      "route");
}

bsg_status bsg_route_noalloc(const float* logits, int64_t T, int E, int k, int renorm,
                             int bin_rows, int32_t* expert_idx, float* gate, int32_t* dest_row,
                             int32_t* counts, int32_t* bin_offsets, bsg_stream_t stream) {
    const bsg_status s =
        check_route(logits, T, E, k, bin_rows, expert_idx, gate, dest_row, counts, bin_offsets);
    if (s != BSG_OK) return s;
    const size_t need = bsg_route_workspace_bytes(T, k, E);
    if (need > BSG_ROUTE_SCRATCH_BYTES)
        return fail(BSG_EUNSUPPORTED,
                    "route_noalloc needs %zu bytes of scratch (ceil(T/64) * E * 4), above its "
                    "static %zu bytes; call bsg_route with a workspace",
                    need, (size_t)BSG_ROUTE_SCRATCH_BYTES);
    int32_t* scratch = nullptr;
    const hipError_t e = bsg::route_scratch((hipStream_t)stream, &scratch);
    if (e != hipSuccess) return hip_status(e, "route_noalloc scratch");
    return hip_status(bsg::launch_route(logits, T, E, k, renorm, bin_rows, expert_idx, gate, dest_row,
                                        counts, bin_offsets, scratch, bsg::TopoJob{},
                                        bsg::PermJob{}, (hipStream_t)stream),
                      "route_noalloc");
}

bsg_status bsg_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                              const int32_t* expert_idx, const int32_t* dest_row, const void* dy,
                              int dy_dtype, int d, const void* yp, int yp_dtype, int64_t ld_yp,
                              float* dlogits, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dy_dtype) && dtype_ok(yp_dtype), "unknown dtype");
    REQUIRE(T >= 1, "T must be positive");
    REQUIRE(E >= 1 && E <= BSG_MAX_EXPERTS, "E must be in [1, %d]", BSG_MAX_EXPERTS);
    REQUIRE(k >= 1 && k <= E, "k must be in [1, E]");
    if (k > BSG_MAX_TOPK) return fail(BSG_EUNSUPPORTED, "k > %d is not implemented", BSG_MAX_TOPK);
    REQUIRE(T <= INT32_MAX && T * k < INT32_MAX, "T*k must fit int32 assignment ids");
    REQUIRE(d >= 1 && d <= kMaxWidth && (d * elt_bytes(dy_dtype)) % 16 == 0 &&
                (d * elt_bytes(yp_dtype)) % 16 == 0,
            "d must keep rows 16-byte aligned");
    REQUIRE(ld_yp >= d && ld_yp <= kMaxLd && (ld_yp * elt_bytes(yp_dtype)) % 16 == 0,
            "ld_yp must be >= d with 16-byte aligned rows");
    REQUIRE_PTR(logits);
    REQUIRE_PTR(expert_idx);
    REQUIRE_PTR(dest_row);
    REQUIRE_VEC_PTR(dy);
    REQUIRE_VEC_PTR(yp);
    REQUIRE_PTR(dlogits);
    return hip_status(bsg::launch_route_backward(logits, T, E, k, renorm, expert_idx, dest_row, dy,
                                                 dy_dtype, d, yp, yp_dtype, ld_yp, dlogits,
                                                 (hipStream_t)stream),
                      "route_backward");
}

bsg_status bsg_permute_pad(const void* x, int dtype, int64_t T, int d, int k,
                           const int32_t* dest_row, const float* scale, const int32_t* counts,
                           const int32_t* bin_offsets, int E, int bin_rows, int64_t Tp_max,
                           int32_t* row_src, void* xp, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype), "unknown dtype %d", dtype);
    const bsg_status bs = check_bin(bin_rows);
    if (bs != BSG_OK) return bs;
    REQUIRE(T >= 1 && k >= 1 && E >= 1 && E <= BSG_MAX_EXPERTS && k <= E, "bad T, k or E");
    REQUIRE(k <= BSG_MAX_TOPK, "k > %d", BSG_MAX_TOPK);
    REQUIRE(T <= INT32_MAX && T * k < INT32_MAX, "T*k must fit int32");
    REQUIRE(d >= 1 && d <= kMaxWidth && (d * elt_bytes(dtype)) % 16 == 0,
            "d must keep rows 16-byte aligned");
    REQUIRE(Tp_max >= bsg_max_padded_rows(T, k, E, bin_rows), "Tp_max below the padded-row bound");
    REQUIRE_VEC_PTR(x);
    REQUIRE_VEC_PTR(xp);
    REQUIRE_PTR(dest_row);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(bin_offsets);
    REQUIRE_PTR(row_src);
    REQUIRE(scale == nullptr || aligned(scale, 4), "scale must be 4-byte aligned");
    return hip_status(bsg::launch_permute_pad(x, dtype, T, d, k, dest_row, scale, counts,
                                              bin_offsets, E, bin_rows, Tp_max, row_src, xp,
                                              (hipStream_t)stream),
                      "permute_pad");
}

bsg_status bsg_permute_pad_gate_backward(const void* dy, int dtype, int64_t T, int d, int k,
                                         const int32_t* dest_row, const float* gate,
                                         const int32_t* counts, const int32_t* bin_offsets, int E,
                                         int bin_rows, int64_t Tp_max, int32_t* row_src,
                                         void* dyp, const float* logits, int renorm,
                                         const int32_t* expert_idx, const void* yp, int yp_dtype,
                                         int64_t ld_yp, float* dlogits, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype) && dtype_ok(yp_dtype), "unknown dtype");
    if (dtype == BSG_F32 && yp_dtype == BSG_BF16)
        return fail(BSG_EUNSUPPORTED, "fp32 dy with bf16 yp is not implemented");
    const bsg_status bs = check_bin(bin_rows);
    if (bs != BSG_OK) return bs;
    REQUIRE(T >= 1 && k >= 1 && E >= 1 && E <= BSG_MAX_EXPERTS && k <= E, "bad T, k or E");
    if (k > BSG_MAX_TOPK) return fail(BSG_EUNSUPPORTED, "k > %d is not implemented", BSG_MAX_TOPK);
    REQUIRE(T <= INT32_MAX && T * k < INT32_MAX, "T*k must fit int32");
    REQUIRE(d >= 1 && d <= kMaxWidth && (d * elt_bytes(dtype)) % 16 == 0,
            "d must keep rows 16-byte aligned");
    REQUIRE(ld_yp >= d && ld_yp <= kMaxLd && (ld_yp * elt_bytes(yp_dtype)) % 16 == 0,
            "ld_yp must be >= d with 16-byte aligned rows");
    REQUIRE(Tp_max >= bsg_max_padded_rows(T, k, E, bin_rows), "Tp_max below the padded-row bound");
    REQUIRE_VEC_PTR(dy);
    REQUIRE_VEC_PTR(dyp);
    REQUIRE_VEC_PTR(yp);
    REQUIRE_PTR(dest_row);
    REQUIRE_PTR(gate);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(bin_offsets);
    REQUIRE_PTR(row_src);
    REQUIRE_PTR(logits);
    REQUIRE_PTR(expert_idx);
    REQUIRE_PTR(dlogits);
    return hip_status(bsg::launch_permute_gate_backward(dy, dtype, T, d, k, dest_row, gate, counts,
                                                        bin_offsets, E, bin_rows, Tp_max, row_src,
                                                        dyp,
                                                        logits, renorm, expert_idx, yp, yp_dtype,
                                                        ld_yp, dlogits, (hipStream_t)stream),
                      "permute_pad_gate_backward");
}

// Tiles go in groups of row pairs (see the kernel's tile order); a group
// pays off when its rows share an expert, so it follows the expected row
// pairs per expert, Tp_max / (256 E): 1, 2 or 4, and 8 when the experts are
// also few (at most 16), so that long bins are the rule rather than the few
// hot experts of a skewed routing: a group of 8 row pairs then stays inside
// one expert, and the tiles an XCD runs at once share each weight panel
// eight ways instead of four.  The topology builder cuts each expert's row
// pairs into groups of at most this many.
static int tile_group(int64_t Tp_max, int E) {
    const int64_t rpe = Tp_max / (2 * BSG_BLOCK * (int64_t)E);
    return (rpe >= 8 && E <= 16) ? 8 : rpe >= 4 ? 4 : rpe >= 2 ? 2 : 1;
}

static bsg_status check_topology_args(int E, int f, int64_t Tp_max, const bsg_topology* topo) {
    REQUIRE(E >= 1 && E <= BSG_MAX_EXPERTS, "E must be in [1, %d]", BSG_MAX_EXPERTS);
    REQUIRE(f >= BSG_BLOCK && f % BSG_BLOCK == 0, "f must be a positive multiple of 128");
    bsg_status s = check_topology(topo);
    if (s != BSG_OK) return s;
    REQUIRE(topo->E == E && topo->F == f / BSG_BLOCK && topo->Tp_max == Tp_max,
            "topo capacity does not match E, f, Tp_max");
    return BSG_OK;
}

// What the topology kernels need of a validated topology.
static bsg::TopoJob topo_job(const bsg_topology* t) {
    bsg::TopoJob j{};
    j.o = bsg::TopoArrays{t->row_ptr, t->col_idx,   t->row_idx,      t->col_ptr,
                          t->trans_idx, t->row_tiles, t->expert_order, t->meta};
    j.F = t->F;
    j.br = t->block_rows;
    j.group = tile_group(t->Tp_max, t->E);
    j.on = 1;
    j.row_blocks_max = t->Tp_max / t->block_rows;
    j.row_tiles_max = row_tiles_max(j.row_blocks_max, t->E, t->block_rows);
    return j;
}

bsg_status bsg_build_topology(const int32_t* bin_offsets, int E, int f, int64_t Tp_max,
                              const bsg_topology* topo, bsg_stream_t stream) {
    REQUIRE_PTR(bin_offsets);
    const bsg_status s = check_topology_args(E, f, Tp_max, topo);
    if (s != BSG_OK) return s;
    const bsg::TopoJob j = topo_job(topo);
    return hip_status(
        bsg::launch_build_topology(bin_offsets, E, j.F, j.br, j.row_blocks_max, j.row_tiles_max,
                                   j.o.row_ptr, j.o.col_idx, j.o.row_idx, j.o.col_ptr,
                                   j.o.trans_idx, j.o.row_tiles, j.o.expert_order, j.o.meta,
                                   j.group, (hipStream_t)stream),
        "build_topology");
}

bsg_status bsg_route_topology(const float* logits, int64_t T, int E, int k, int renorm,
                              int bin_rows, int32_t* expert_idx, float* gate, int32_t* dest_row,
                              int32_t* counts, int32_t* bin_offsets, void* workspace,
                              size_t workspace_bytes, int f, int64_t Tp_max,
                              const bsg_topology* topo, bsg_stream_t stream) {
    bsg_status s =
        check_route(logits, T, E, k, bin_rows, expert_idx, gate, dest_row, counts, bin_offsets);
    if (s != BSG_OK) return s;
    REQUIRE_PTR(workspace);
    REQUIRE(workspace_bytes >= bsg_route_workspace_bytes(T, k, E), "workspace too small (%zu < %zu)",
            workspace_bytes, bsg_route_workspace_bytes(T, k, E));
    if ((s = check_topology_args(E, f, Tp_max, topo)) != BSG_OK) return s;
    return hip_status(bsg::launch_route(logits, T, E, k, renorm, bin_rows, expert_idx, gate, dest_row,
                                        counts, bin_offsets, (int32_t*)workspace, topo_job(topo),
                                        bsg::PermJob{}, (hipStream_t)stream),
                      "route_topology");
}

bsg_status bsg_route_permute_topology(const float* logits, int64_t T, int E, int k, int renorm,
                                      int bin_rows, int32_t* expert_idx, float* gate,
                                      int32_t* dest_row, int32_t* counts, int32_t* bin_offsets,
                                      void* workspace, size_t workspace_bytes, const void* x,
                                      int dtype, int d, int64_t Tp_max, int32_t* row_src,
                                      void* xp, int f, const bsg_topology* topo,
                                      bsg_stream_t stream) {
    bsg_status s =
        check_route(logits, T, E, k, bin_rows, expert_idx, gate, dest_row, counts, bin_offsets);
    if (s != BSG_OK) return s;
    REQUIRE_PTR(workspace);
    REQUIRE(workspace_bytes >= bsg_route_workspace_bytes(T, k, E), "workspace too small (%zu < %zu)",
            workspace_bytes, bsg_route_workspace_bytes(T, k, E));
    // the permutation's rules (bsg_permute_pad's, without a scale)
    REQUIRE(dtype_ok(dtype), "unknown dtype %d", dtype);
    REQUIRE(d >= 1 && d <= kMaxWidth && (d * elt_bytes(dtype)) % 16 == 0,
            "d must keep rows 16-byte aligned");
    REQUIRE(Tp_max >= bsg_max_padded_rows(T, k, E, bin_rows), "Tp_max below the padded-row bound");
    REQUIRE_VEC_PTR(x);
    REQUIRE_VEC_PTR(xp);
    REQUIRE_PTR(row_src);
    if (topo != nullptr && (s = check_topology_args(E, f, Tp_max, topo)) != BSG_OK) return s;
    bsg::PermJob pj{};
    pj.x = x;
    pj.xp = xp;
    pj.row_src = row_src;
    pj.chunks = d * elt_bytes(dtype) / 16;
    pj.on = 1;
    pj.Tp_max = Tp_max;
    return hip_status(bsg::launch_route(logits, T, E, k, renorm, bin_rows, expert_idx, gate, dest_row,
                                        counts, bin_offsets, (int32_t*)workspace,
                                        topo ? topo_job(topo) : bsg::TopoJob{}, pj,
                                        (hipStream_t)stream),
                      "route_permute_topology");
}

// Compute units of the stream's device, looked up once per device.
static hipError_t device_cus(hipStream_t stream, int* ncu) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cus[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        if (n <= 0) return hipErrorInvalidDevice;
        cus[dev] = n;
    }
    *ncu = cus[dev];
    return hipSuccess;
}

static bsg::GemmParams gemm_params(const bsg_topology* t) {
    bsg::GemmParams p{};
    p.col_idx = t->col_idx;
    p.col_ptr = t->col_ptr;
    p.row_tiles = t->row_tiles;
    p.expert_order = t->expert_order;
    p.meta = t->meta;
    p.E = t->E;
    p.F = t->F;
    p.br = t->block_rows;
    p.group = tile_group(t->Tp_max, t->E);
    return p;
}

static int64_t tiles_max(const bsg_topology* t) {
    return row_tiles_max(t->Tp_max / t->block_rows, t->E, t->block_rows);
}

bsg_status bsg_sdd(const void* a, int64_t lda, const void* b, const void* b2, int64_t ldb,
                   int trans_b, int K, const bsg_topology* topo, int epilogue, const void* aux_in,
                   void* out_blocks, void* aux_out, int dtype, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype), "unknown dtype %d", dtype);
    bsg_status s = check_topology(topo);
    if (s != BSG_OK) return s;
    REQUIRE(epilogue >= BSG_EPI_NONE && epilogue <= BSG_EPI_SILU_MUL_BWD, "unknown epilogue %d",
            epilogue);
    const int es = elt_bytes(dtype);
    const int kt = dtype == BSG_BF16 ? 64 : 32;
    const int64_t ncol = (int64_t)topo->E * topo->F * BSG_BLOCK;
    REQUIRE(K >= kt && K % kt == 0, "K must be a positive multiple of %d", kt);
    REQUIRE(lda >= K && lda <= kMaxLd && (lda * es) % 16 == 0,
            "lda must be >= K with 16-byte aligned rows");
    REQUIRE(trans_b == 0 || trans_b == 1, "trans_b must be 0 or 1");
    REQUIRE(ldb >= (trans_b ? K : ncol) && ldb <= kMaxLd && (ldb * es) % 16 == 0,
            "ldb too small or rows not 16-byte aligned");
    REQUIRE_PANEL_LD(lda, es, true);
    REQUIRE_PANEL_LD(ldb, es, trans_b == 1);
    REQUIRE_VEC_PTR(a);
    REQUIRE_VEC_PTR(b);
    REQUIRE_VEC_PTR(out_blocks);
    if (epilogue == BSG_EPI_SILU_MUL) {
        REQUIRE_VEC_PTR(b2);
        if (trans_b) return fail(BSG_EUNSUPPORTED, "SILU_MUL with trans_b is not implemented");
    } else {
        REQUIRE(b2 == nullptr, "b2 is only used by BSG_EPI_SILU_MUL");
    }
    if (epilogue == BSG_EPI_GELU_BWD || epilogue == BSG_EPI_SILU_MUL_BWD) REQUIRE_VEC_PTR(aux_in);
    else REQUIRE(aux_in == nullptr, "aux_in is only used by the backward epilogues");
    if (epilogue != BSG_EPI_GELU && epilogue != BSG_EPI_SILU_MUL)
        REQUIRE(aux_out == nullptr, "aux_out is only used by BSG_EPI_GELU and BSG_EPI_SILU_MUL");
    else REQUIRE(aux_out == nullptr || aligned(aux_out, 16), "aux_out must be 16-byte aligned");
    bsg::GemmParams p = gemm_params(topo);
    p.a = a;
    p.b = b;
    p.b2 = b2;
    p.aux_in = aux_in;
    p.out = out_blocks;
    p.aux_out = aux_out;
    p.plane = (topo->Tp_max / topo->block_rows) * topo->F * topo->block_rows * BSG_BLOCK;
    p.lda = lda;
    p.ldb = ldb;
    p.K = K;
    // the compute units size the split of a sparse last round
    const hipError_t e = device_cus((hipStream_t)stream, &p.ncu);
    if (e != hipSuccess) return hip_status(e, "sdd");
    return hip_status(bsg::launch_sdd(p, tiles_max(topo), trans_b,
                                      epilogue, dtype, (hipStream_t)stream),
                      "sdd");
}

bsg_status bsg_dsd_workspace_bytes(bsg_stream_t stream, int64_t* bytes) {
    REQUIRE(bytes != nullptr, "bytes is NULL");
    int ncu = 0;
    const hipError_t e = device_cus((hipStream_t)stream, &ncu);
    if (e != hipSuccess) return hip_status(e, "dsd_workspace_bytes");
    *bytes = (int64_t)ncu * bsg::kSplitShareBytes;
    return ok();
}

bsg_status bsg_dsd(const void* blocks, const void* blocks2, const bsg_topology* topo,
                   const void* b, const void* b2, int64_t ldb, int trans_b, int N, void* c,
                   int64_t ldc, int c_dtype, int dtype, void* workspace, size_t workspace_bytes,
                   bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype) && dtype_ok(c_dtype), "unknown dtype");
    if (dtype == BSG_F32 && c_dtype != BSG_F32)
        return fail(BSG_EUNSUPPORTED, "fp32 operands need an fp32 output");
    bsg_status s = check_topology(topo);
    if (s != BSG_OK) return s;
    const int es = elt_bytes(dtype), ces = elt_bytes(c_dtype);
    const int64_t ncol = (int64_t)topo->E * topo->F * BSG_BLOCK;
    REQUIRE(N >= BSG_BLOCK && N <= kMaxWidth && N % BSG_BLOCK == 0,
            "N must be a positive multiple of 128");
    REQUIRE(trans_b == 0 || trans_b == 1, "trans_b must be 0 or 1");
    REQUIRE(ldb >= (trans_b ? ncol : N) && ldb <= kMaxLd && (ldb * es) % 16 == 0,
            "ldb too small or rows not 16-byte aligned");
    REQUIRE(ldc >= N && ldc <= kMaxLd && (ldc * ces) % 16 == 0,
            "ldc must be >= N with 16-byte aligned rows");
    REQUIRE_PANEL_LD(ldb, es, trans_b == 1);
    REQUIRE_VEC_PTR(blocks);
    REQUIRE_VEC_PTR(b);
    REQUIRE_VEC_PTR(c);
    REQUIRE((blocks2 == nullptr) == (b2 == nullptr), "blocks2 and b2 go together");
    if (blocks2) {
        REQUIRE_VEC_PTR(blocks2);
        REQUIRE_VEC_PTR(b2);
        REQUIRE((int64_t)topo->E * topo->F < bsg::kSecondSet, "too many column blocks");
    }
    if (workspace) {
        REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
        REQUIRE(workspace_bytes >= 2 * (size_t)bsg::kSplitShareBytes,
                "workspace too small (%zu < %d): two tile shares at least", workspace_bytes,
                2 * bsg::kSplitShareBytes);
    }
    bsg::GemmParams p = gemm_params(topo);
    p.a = blocks;
    p.a2 = blocks2;
    p.b = b;
    p.b2 = b2;
    p.out = c;
    p.ldb = ldb;
    p.ldc = ldc;
    p.N = N;
    p.ntn = (N + 255) / 256;
    // the last round's split: only tiles of at least kSplitMinBlocks K-blocks
    if (workspace && (int64_t)topo->F * (blocks2 ? 2 : 1) >= bsg::kSplitMinBlocks) {
        int ncu = 0;
        const hipError_t e = device_cus((hipStream_t)stream, &ncu);
        if (e != hipSuccess) return hip_status(e, "dsd");
        p.ws = (float*)workspace;
        p.ws_units = (int)std::min<size_t>(workspace_bytes / bsg::kSplitShareBytes, INT32_MAX);
        p.ncu = ncu;
    }
    return hip_status(bsg::launch_dsd(p, tiles_max(topo), trans_b,
                                      c_dtype, dtype, (hipStream_t)stream),
                      "dsd");
}

bsg_status bsg_dsd_combine_top1(const void* blocks, const bsg_topology* topo, const void* b,
                                int64_t ldb, int trans_b, int N, void* c, int64_t ldc,
                                const int32_t* row_src, const float* gate, void* y, int64_t ldy,
                                int dtype, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype), "unknown dtype %d", dtype);
    if (dtype != BSG_BF16) return fail(BSG_EUNSUPPORTED, "dsd_combine_top1 is implemented for bf16");
    bsg_status s = check_topology(topo);
    if (s != BSG_OK) return s;
    const int64_t ncol = (int64_t)topo->E * topo->F * BSG_BLOCK;
    REQUIRE(N >= BSG_BLOCK && N <= kMaxWidth && N % BSG_BLOCK == 0,
            "N must be a positive multiple of 128");
    REQUIRE(trans_b == 0 || trans_b == 1, "trans_b must be 0 or 1");
    REQUIRE(ldb >= (trans_b ? ncol : N) && ldb <= kMaxLd && (ldb * 2) % 16 == 0,
            "ldb too small or rows not 16-byte aligned");
    REQUIRE(ldy >= N && ldy <= kMaxLd && (ldy * 2) % 16 == 0,
            "ldy must be >= N with 16-byte aligned rows");
    REQUIRE_PANEL_LD(ldb, 2, trans_b == 1);
    REQUIRE_VEC_PTR(blocks);
    REQUIRE_VEC_PTR(b);
    REQUIRE_VEC_PTR(y);
    REQUIRE_PTR(row_src);
    REQUIRE(gate == nullptr || aligned(gate, 4), "gate must be 4-byte aligned");
    if (c) {
        REQUIRE(aligned(c, 16), "c must be 16-byte aligned");
        REQUIRE(ldc >= N && ldc <= kMaxLd && (ldc * 2) % 16 == 0,
                "ldc must be >= N with 16-byte aligned rows");
    }
    bsg::GemmParams p = gemm_params(topo);
    p.a = blocks;
    p.b = b;
    p.out = c;
    p.ldb = ldb;
    p.ldc = ldc;
    p.N = N;
    p.ntn = (N + 255) / 256;
    p.scat_rows = row_src;
    p.scat_gate = gate;
    p.scat_out = y;
    p.scat_ld = ldy;
    return hip_status(bsg::launch_dsd(p, tiles_max(topo), trans_b,
                                      BSG_BF16, BSG_BF16, (hipStream_t)stream),
                      "dsd_combine_top1");
}

bsg_status bsg_dstd(const void* blocks, const bsg_topology* topo, const void* dmat, int64_t ldd,
                    int N, void* c, int64_t ldc, int trans_c, int dtype, bsg_stream_t stream) {
    REQUIRE(dtype_ok(dtype), "unknown dtype %d", dtype);
    bsg_status s = check_topology(topo);
    if (s != BSG_OK) return s;
    const int es = elt_bytes(dtype);
    const int64_t ncol = (int64_t)topo->E * topo->F * BSG_BLOCK;
    REQUIRE(N >= BSG_BLOCK && N <= kMaxWidth && N % BSG_BLOCK == 0,
            "N must be a positive multiple of 128");
    REQUIRE(trans_c == 0 || trans_c == 1, "trans_c must be 0 or 1");
    REQUIRE(ldd >= N && ldd <= kMaxLd && (ldd * es) % 16 == 0,
            "ldd must be >= N with 16-byte aligned rows");
    REQUIRE(ldc >= (trans_c ? ncol : N) && ldc <= kMaxLd && (ldc * es) % 16 == 0,
            "ldc too small or rows not 16-byte aligned");
    REQUIRE_PANEL_LD(ldd, es, false);
    REQUIRE_VEC_PTR(blocks);
    REQUIRE_VEC_PTR(dmat);
    REQUIRE_VEC_PTR(c);
    bsg::GemmParams p = gemm_params(topo);
    p.a = blocks;
    p.b = dmat;
    p.out = c;
    p.ldb = ldd;
    p.ldc = ldc;
    p.N = N;
    p.ntn = (N + 255) / 256;
    return hip_status(bsg::launch_dstd(p, trans_c, dtype, (hipStream_t)stream), "dstd");
}

bsg_status bsg_unpermute_combine(const void* yp, int yp_dtype, int64_t ld_yp,
                                 const int32_t* dest_row, const float* gate, int64_t T, int k,
                                 int d, void* y, int y_dtype, bsg_stream_t stream) {
    REQUIRE(dtype_ok(yp_dtype) && dtype_ok(y_dtype), "unknown dtype");
    REQUIRE(T >= 1 && T <= INT32_MAX && k >= 1 && k <= BSG_MAX_TOPK && T * k < INT32_MAX,
            "bad T or k");
    REQUIRE(d >= 8 && d <= kMaxWidth && d % 8 == 0, "d must be a positive multiple of 8");
    REQUIRE(ld_yp >= d && ld_yp <= kMaxLd && (ld_yp * elt_bytes(yp_dtype)) % 16 == 0,
            "ld_yp must be >= d with 16-byte aligned rows");
    REQUIRE_VEC_PTR(yp);
    REQUIRE_VEC_PTR(y);
    REQUIRE_PTR(dest_row);
    REQUIRE(gate == nullptr || aligned(gate, 4), "gate must be 4-byte aligned");
    return hip_status(bsg::launch_unpermute_combine(yp, yp_dtype, ld_yp, dest_row, gate, T, k, d,
                                                    y, y_dtype, (hipStream_t)stream),
                      "unpermute_combine");
}

bsg_status bsg_stream_copy(const void* src, void* dst, size_t bytes, bsg_stream_t stream) {
    REQUIRE_VEC_PTR(src);
    REQUIRE_VEC_PTR(dst);
    REQUIRE(bytes % 16 == 0 && bytes <= ((size_t)1 << 46), "bytes must be a multiple of 16");
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    REQUIRE(s + bytes <= d || d + bytes <= s, "src and dst overlap");
    return hip_status(bsg::launch_stream_copy(src, dst, (int64_t)(bytes / 16), (hipStream_t)stream),
                      "stream_copy");
}

}  // extern "C"
