// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

constexpr int kF32 = 0;   // matches BSG_F32
constexpr int kBf16 = 1;  // matches BSG_BF16

constexpr int kEpiNone = 0;
constexpr int kEpiGelu = 1;
constexpr int kEpiSiluMul = 2;
constexpr int kEpiGeluBwd = 3;
constexpr int kEpiSiluMulBwd = 4;
constexpr int kEpiGeluSave = 5;     // internal: GeLU that also stores its derivative
constexpr int kEpiSiluMulSave = 6;  // internal: SiLU*mul that also stores silu, u*silu'
constexpr int kEpiScatter = 7;      // internal: DSD rows also written in token order (top-1)

constexpr int kModeSdd = 0;
constexpr int kModeSddOne = 1;
constexpr int kModeDsd = 2;
constexpr int kModeDstd = 3;
constexpr int kModeDsd2 = 4;  // DSD over two block sets, each with its own B

// DSD over two block sets: the staged weight-row index of a K-block of the
// second set carries this bit
constexpr int kSecondSet = 1 << 30;

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kRouteChunk = 64;  // tokens per routing chunk

// A DSD's split last round: one share holds the fp32 partial sums of one
// 256 x 256 tile; a tile is split only when it walks at least this many
// K-blocks (shorter tiles do not repay the shares' traffic).
constexpr int kSplitShareBytes = 256 * 256 * 4;
constexpr int kSplitMinBlocks = 32;

struct GemmParams {
    const void* a;       // SDD: dense rows; DSD / DSTD: sparse blocks
    const void* a2;      // two-set DSD: the second block set
    const void* b;       // SDD / DSD: dense B; DSTD: dense rows (dmat)
    const void* b2;      // SDD dual-B second operand (SwiGLU up projection);
                         // two-set DSD: the second set's B
    const void* aux_in;  // SDD GELU_BWD: saved GeLU derivative blocks;
                         // SILU_MUL_BWD: the two saved planes (silu, u*silu')
    void* out;           // SILU_MUL_BWD: two planes (gate, up gradients)
    void* aux_out;       // SDD GELU: optional saved derivative blocks;
                         // SILU_MUL: optional two planes (silu, u*silu')
    int64_t plane;       // elements between the planes of a two-plane block array
    // DSD with top-1 routing: rows also go to token order, y[row_src[r]] =
    // rd(gate[row_src[r]] * rd(c[r])) (gate NULL: 1); out may then be NULL
    const int32_t* scat_rows;
    const float* scat_gate;
    void* scat_out;
    int64_t scat_ld;
    int64_t lda, ldb, ldc;
    // the topology (its block pointer, row and transpose index lists are
    // closed forms of col_idx and col_ptr, which the kernels compute)
    const int32_t* col_idx;
    const int32_t* col_ptr;
    const int32_t* row_tiles;  // tiles of up to 256 rows of one expert (block rows sharing a
                               // column list)
    const int32_t* expert_order;  // experts by descending row count
    const int32_t* meta;  // {nnz, R, overflow, row pairs} written by build_topology
    int K;                // SDD reduction length
    int N;                // DSD / DSTD output width
    int ntn;              // 256-wide output tiles along N
    int E, F;             // experts, column blocks per expert
    int br;               // rows of a block: 128, or 64 for bins of 64 rows
    int group;            // DSTD: column pairs per group of an expert's tiles (>= 1); SDD and
                          // DSD take their groups from row_tiles
    // DSD (plain epilogue): workspace for the split of the last round (NULL:
    // no split), in shares of one tile's fp32 partial sums (256 KB each), and
    // the GPU's compute units
    float* ws;
    int ws_units;
    int ncu;
};

// The arrays of a topology (bsg_topology's device pointers).
struct TopoArrays {
    int32_t *row_ptr, *col_idx, *row_idx, *col_ptr, *trans_idx, *row_tiles, *expert_order, *meta;
};

// A topology for the routing to build in its placement launch, from the bin
// offsets it has just formed (on = 0: none).  Fields as launch_build_topology.
struct TopoJob {
    TopoArrays o;
    int F, br, group, on;
    int64_t row_blocks_max, row_tiles_max;
};

// A permutation for the routing to do in its placement launch (what
// launch_permute_pad does with no scale): each placing workgroup copies the
// rows of the tokens it has just placed (on = 0: none).
struct PermJob {
    const void* x;     // [T, chunks] 16-byte chunks
    void* xp;          // [Tp_max, chunks]
    int32_t* row_src;  // [Tp_max]
    int chunks;        // 16-byte chunks per row
    int on;
    int64_t Tp_max;
};

// Bytes of the file-scope device array behind the allocation-free routing
// entry point (per GPU): 4 MiB, one count per (64-token chunk, expert).
constexpr size_t kRouteScratchBytes = size_t(4) << 20;

// That array's address on the device of `stream` (looked up once per device).
hipError_t route_scratch(hipStream_t stream, int32_t** out);

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renorm, int bin_rows,
                        int32_t* expert_idx, float* gate, int32_t* dest_row, int32_t* counts,
                        int32_t* bin_offsets, int32_t* workspace, const TopoJob& topo,
                        const PermJob& perm, hipStream_t stream);

hipError_t launch_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                                 const int32_t* expert_idx, const int32_t* dest_row,
                                 const void* dy, int dy_dtype, int d, const void* yp,
                                 int yp_dtype, int64_t ld_yp, float* dlogits, hipStream_t stream);

hipError_t launch_permute_pad(const void* x, int dtype, int64_t T, int d, int k,
                              const int32_t* dest_row, const float* scale, const int32_t* counts,
                              const int32_t* bin_offsets, int E, int bin_rows, int64_t Tp_max,
                              int32_t* row_src, void* xp, hipStream_t stream);

hipError_t launch_permute_gate_backward(const void* dy, int dtype, int64_t T, int d, int k,
                                        const int32_t* dest_row, const float* gate,
                                        const int32_t* counts, const int32_t* bin_offsets, int E,
                                        int bin_rows, int64_t Tp_max, int32_t* row_src,
                                        void* dyp,
                                        const float* logits, int renorm,
                                        const int32_t* expert_idx, const void* yp, int yp_dtype,
                                        int64_t ld_yp, float* dlogits, hipStream_t stream);

hipError_t launch_build_topology(const int32_t* bin_offsets, int E, int F, int br,
                                 int64_t row_blocks_max, int64_t row_tiles_max, int32_t* row_ptr,
                                 int32_t* col_idx, int32_t* row_idx, int32_t* col_ptr,
                                 int32_t* trans_idx, int32_t* row_tiles, int32_t* expert_order,
                                 int32_t* meta, int group, hipStream_t stream);

hipError_t launch_sdd(const GemmParams& p, int64_t row_tiles_max, int trans_b, int epi, int dtype,
                      hipStream_t s);
hipError_t launch_dsd(const GemmParams& p, int64_t row_tiles_max, int trans_b, int c_dtype,
                      int dtype, hipStream_t s);
hipError_t launch_dstd(const GemmParams& p, int trans_c, int dtype, hipStream_t s);

hipError_t launch_unpermute_combine(const void* yp, int yp_dtype, int64_t ld_yp,
                                    const int32_t* dest_row, const float* gate, int64_t T, int k,
                                    int d, void* y, int y_dtype, hipStream_t stream);

hipError_t launch_stream_copy(const void* src, void* dst, int64_t words, hipStream_t stream);

}  // namespace bsg
