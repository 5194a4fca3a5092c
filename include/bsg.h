/*
 * bsg.h - C ABI of the MI355X (gfx950) dropless-MoE block-sparse expert layer.
 *
 * The layer follows the MegaBlocks formulation described in George Lin's
 * Blog (post on MegaBlocks and FlexMoE, part 1): the expert MLP over a
 * variable number of tokens per expert is one block-sparse product with
 * 128x128 blocks (section 1.2), SDD for the first layer, the activation,
 * DSD for the second layer, and DSTD for the weight gradients through a
 * transpose index (section 1.3); routing, a fused permutation + padding
 * kernel and a one-launch topology builder come first (section 1.4).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer unless stated otherwise,
 *    allocated and freed by the caller; the library never allocates, frees,
 *    synchronises the host or keeps global mutable state (one exception:
 *    the static device array of bsg_route_noalloc).
 *  - Every kernel is enqueued on `stream` (a hipStream_t; NULL means the
 *    null stream) and runs asynchronously; results are valid once the
 *    stream has reached them.
 *  - Arrays of activations, weights and blocks are moved with 16-byte
 *    vectors and must be 16-byte aligned; index, count and gate arrays
 *    must be 4-byte aligned.  Leading dimensions are in elements and must
 *    keep every row 16-byte aligned.  The products (sdd, dsd, dstd) reach
 *    the rows of an operand panel through 32-bit byte offsets from the
 *    panel's first row: a dense operand's leading dimension must keep
 *    127 * ld * elt + 64 (rows contiguous along K) or 31 * ld * 2 + 256
 *    (bf16) / 15 * ld * 4 + 512 (fp32) (rows contiguous along M or N)
 *    below 2^32, else BSG_EUNSUPPORTED.
 *  - Arguments are validated BEFORE any HIP call.  An invalid argument
 *    returns BSG_EINVAL, a valid but unimplemented combination
 *    BSG_EUNSUPPORTED, a failed launch BSG_EHIP; bsg_last_error() then
 *    describes the failure (per thread).  Faults inside a kernel surface at
 *    the caller's next synchronisation.
 *  - Sizes that depend on the routing (Tp, the number of nonzero blocks) are
 *    produced on the device; buffers are sized for their upper bounds from
 *    the size queries below, so no call needs a host round trip.
 *  - dtype codes: BSG_F32 (fp32) or BSG_BF16 (bf16 storage, fp32
 *    accumulation).
 *
 * Symbols: T tokens, d model width, E experts, f per-expert hidden width,
 * k experts per token, F = f/128 column blocks per expert, A = T*k
 * assignments, Tp = padded row count, BR = block rows (128, the block of
 * section 1.3, or 64 for the block-size study), R = Tp/BR row blocks,
 * nnz = R*F nonzero blocks of BR x 128.
 */
#ifndef BSG_H
#define BSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSG_OK = 0,
    BSG_EINVAL = -1,       /* null pointer, bad size, misaligned pointer, bad code */
    BSG_EUNSUPPORTED = -2, /* valid request the library does not implement */
    BSG_EHIP = -3          /* the HIP runtime rejected a launch */
} bsg_status;

typedef enum { BSG_F32 = 0, BSG_BF16 = 1 } bsg_dtype;

typedef enum {
    BSG_EPI_NONE = 0,        /* out = acc */
    BSG_EPI_GELU = 1,        /* out = gelu(acc) (exact erf form); optional aux_out = gelu'(acc) */
    BSG_EPI_SILU_MUL = 2,    /* dual B: out = silu(acc_b) * acc_b2; optional aux_out planes
                                silu(acc_b), acc_b2 * silu'(acc_b) */
    BSG_EPI_GELU_BWD = 3,    /* out = acc * aux_in (aux_in = saved gelu') */
    BSG_EPI_SILU_MUL_BWD = 4 /* out planes acc * aux_in[1], acc * aux_in[0] */
} bsg_epilogue;

/* A hipStream_t passed as an opaque pointer (NULL = null stream). */
typedef void* bsg_stream_t;

#define BSG_BLOCK 128
#define BSG_MAX_EXPERTS 1024
#define BSG_MAX_TOPK 32

/* Upper bounds for the topology arrays (pure host function results). */
typedef struct {
    int64_t row_blocks_max; /* Tp_max / BR                                */
    int64_t nnz_max;        /* row_blocks_max * F                         */
    int64_t n_cols;         /* E * F column blocks                        */
    int64_t row_tiles_max;  /* (row_blocks_max + (Q - 1) * (min(E, row_blocks_max) + 1)) / Q,
                               Q = 256 / BR block rows per tile          */
} bsg_topo_sizes;

/*
 * Hybrid BCSR-COO topology of the first layer's output, a [Tp x E*f]
 * matrix of BR x 128 blocks (BR = block_rows: 128, the block of section
 * 1.3, or 64 for the block-size study, whose bins of 64 rows cannot share a
 * 128-row block) where block (r, c) is nonzero when row block r lies in the
 * bin of the expert that owns column block c (section 1.3, "hybrid BCSR-COO
 * format" and "transpose indices").  All arrays are caller-allocated device
 * int32 arrays of the stated capacity:
 *   row_ptr   [row_blocks_max + 1] BCSR block pointer; entries past R hold nnz
 *   col_idx   [nnz_max]  global column block of each block, BCSR order
 *   row_idx   [nnz_max]  materialised row block of each block (COO half)
 *   col_ptr   [E*F + 1]  start of each column's run in trans_idx
 *   trans_idx [nnz_max]  BCSR block ids listed column by column,
 *                        ascending row inside a column (no data copied)
 *   row_tiles [row_tiles_max] the schedule of the products: each
 *                        expert's block rows taken 256 rows at a time
 *                        (Q = 256 / BR consecutive block rows, fewer at
 *                        the expert's end), each expert's tiles cut into
 *                        groups of G = 1, 2, 4 or 8 (the last one
 *                        shorter), G set from Tp_max and E; entry =
 *                        (first block row << 8) | ((group size - 1) << 5)
 *                        | (place in the group << 2) | (block rows - 1)
 *   expert_order [E]     the experts in descending order of their row
 *                        blocks (ties: lower id first), the order in which
 *                        dstd schedules its tiles (longest first)
 *   meta      [4]        written on the device: {nnz, R, status, tiles};
 *                        status = 1 when the routing needs more than
 *                        Tp_max rows, 2 when a bin offset is not a
 *                        multiple of BR: the topology is then published
 *                        empty (nnz = R = 0, all pointers 0) and every
 *                        product writes nothing, or zeros for dstd
 * E, F, block_rows and Tp_max are host values describing the capacity.
 * The products read col_idx, col_ptr, row_tiles, expert_order and meta;
 * the entries of row_ptr (r F), row_idx and trans_idx are closed forms on
 * this block-diagonal structure, which the products compute, so a topology
 * handed to them must have that structure (any bsg_build_topology output
 * has).
 * Sparse operands ("blocks") are stored block-major, [nnz_max][BR][128],
 * each block row-major, in BCSR order.  A two-plane block array is
 * [2][nnz_max][BR][128] with nnz_max = (Tp_max / BR) * F: plane 1 starts
 * nnz_max blocks after plane 0.
 */
typedef struct {
    int32_t* row_ptr;
    int32_t* col_idx;
    int32_t* row_idx;
    int32_t* col_ptr;
    int32_t* trans_idx;
    int32_t* row_tiles;
    int32_t* expert_order;
    int32_t* meta;
    int32_t E;
    int32_t F;
    int32_t block_rows; /* BR: 128, or 64 for bins of 64 rows */
    int64_t Tp_max;
} bsg_topology;

/* ------------------------------------------------------------ size queries */

/* Upper bound on Tp for any routing with bins padded to a multiple of
 * bin_rows (128, the block of section 1.3, or 64 or 256 for the block-size
 * study):
 *   bin_rows * floor((A + (bin_rows - 1) * min(E, A)) / bin_rows),  A = T*k
 * (each non-empty expert pads by at most bin_rows - 1 rows).  Returns -1 on
 * invalid sizes or an unsupported bin_rows. */
int64_t bsg_max_padded_rows(int64_t T, int k, int E, int bin_rows);

/* Capacities of the topology arrays for Tp_max padded rows in blocks of
 * block_rows (128 or 64) rows.  A host-side helper for sizing the caller's
 * buffers; the pages define no such call (the capacities follow from the
 * block grid of section 1.3: Tp_max/BR row blocks of F blocks each, E*F
 * column blocks). */
bsg_status bsg_topology_sizes(int64_t Tp_max, int E, int f, int block_rows,
                              bsg_topo_sizes* out /* host */);

/* Bytes of device workspace bsg_route needs (0 on invalid sizes): per-chunk
 * expert counts of the deterministic placement (64 tokens a chunk).  A
 * host-side helper the pages do not define. */
size_t bsg_route_workspace_bytes(int64_t T, int k, int E);

/* ------------------------------------------------------------------ calls */

/*
 * route - gate + router (section 1.4: tokens are routed, then regrouped by
 * expert; the pages leave the gate's form open, see the design notes).
 *   logits      [T, E] fp32 row-major, finite values.
 *   For each token the k largest logits are picked (ties: lower expert id),
 *   in rank order: expert_idx [T*k] int32, slot j of token t at t*k + j.
 *   gate [T*k] fp32 = softmax over all E logits of the picked expert;
 *   renorm != 0 divides by the sum over the k picks.
 *   counts [E] int32 tokens per expert; bin_offsets [E+1] int32 exclusive
 *   scan of ceil(counts/bin_rows)*bin_rows in ascending expert id
 *   (Tp = bin_offsets[E]).  bin_rows is 128 (section 1.3's padding to the
 *   block), or 64 or 256 (finer and coarser bins for the block-size study;
 *   bins of 64 rows need a topology of 64-row blocks).
 *   dest_row [T*k] int32: row of the padded, expert-grouped layout that
 *   assignment a = t*k + j occupies; inside a bin, ascending a.
 *   workspace: bsg_route_workspace_bytes(T, k, E) device bytes.
 *   Requires 1 <= k <= min(E, 32), 1 <= E <= 1024, T >= 1.
 *   Deterministic: integer results are bit-identical on every run.
 */
bsg_status bsg_route(const float* logits, int64_t T, int E, int k, int renorm, int bin_rows,
                     int32_t* expert_idx, float* gate, int32_t* dest_row, int32_t* counts,
                     int32_t* bin_offsets, void* workspace, size_t workspace_bytes,
                     bsg_stream_t stream);

/*
 * route_noalloc - bsg_route for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the
 * per-chunk expert counts kept in a file-scope device array of the library
 * (BSG_ROUTE_SCRATCH_BYTES per GPU, held until the process ends) instead
 * of a caller workspace.  The call allocates and frees nothing.  Arguments,
 * outputs and limits as bsg_route; in addition
 * bsg_route_workspace_bytes(T, k, E) must not exceed BSG_ROUTE_SCRATCH_BYTES
 * (ceil(T/64) * E <= 1M, e.g. T = 65536 with E = 1024), else
 * BSG_EUNSUPPORTED.  The array's address on the stream's device is looked
 * up on the first call there (BSG_EHIP if that fails).  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Nothing
 * in the array needs clearing: each call writes every count it reads.
 */
#define BSG_ROUTE_SCRATCH_BYTES (4u << 20)
bsg_status bsg_route_noalloc(const float* logits, int64_t T, int E, int k, int renorm,
                             int bin_rows, int32_t* expert_idx, float* gate, int32_t* dest_row,
                             int32_t* counts, int32_t* bin_offsets, bsg_stream_t stream);

/*
 * route_backward - gradient of <dy, y> with respect to the router logits for
 * the gate of bsg_route (plain calculus on it; the top-k selection is held
 * fixed, it passes no gradient):
 *   dg_j = sum_m dy[t][m] * yp[dest_row[t*k + j]][m]
 *   dL/dp[e_j] = dg_j, or with renorm dg_j / S - (sum_i dg_i p[e_i]) / S^2
 *                (S = sum_i p[e_i]); 0 for experts not picked
 *   dlogits[t][e] = p[e] * (dL/dp[e] - sum_u p[u] dL/dp[u]),  p = softmax
 *   logits [T, E] fp32 (as given to bsg_route); expert_idx, dest_row [T*k]
 *   from bsg_route; dy [T, d] (dy_dtype) the gradient of the combined output
 *   y; yp [Tp_max, ld_yp] (yp_dtype) the expert outputs the forward combined;
 *   dlogits [T, E] fp32 out.  fp32 arithmetic.  Same limits as bsg_route.
 */
bsg_status bsg_route_backward(const float* logits, int64_t T, int E, int k, int renorm,
                              const int32_t* expert_idx, const int32_t* dest_row, const void* dy,
                              int dy_dtype, int d, const void* yp, int yp_dtype, int64_t ld_yp,
                              float* dlogits, bsg_stream_t stream);

/*
 * permute_pad - fused permutation + padding (section 1.4 and the padding
 * paragraph of section 1.3): row dest_row[a] of xp receives row a/k of x,
 * times scale[a] when scale is not NULL (the product is rounded once to the
 * dtype); the rows of each bin past its count are zero-filled; row_src
 * receives, for every row below Tp, the assignment that fills it or -1.
 *   x [T, d] (dtype), xp [Tp_max, d] (dtype), row_src [Tp_max] int32,
 *   counts/bin_offsets as produced by bsg_route with the same bin_rows.
 *   Rows >= Tp are untouched, and no row at or beyond Tp_max is written
 *   whatever bin_offsets holds.  d must be a positive multiple of 8 (bf16) or
 *   4 (fp32); Tp_max at least bsg_max_padded_rows(T, k, E, bin_rows).
 */
bsg_status bsg_permute_pad(const void* x, int dtype, int64_t T, int d, int k,
                           const int32_t* dest_row, const float* scale, const int32_t* counts,
                           const int32_t* bin_offsets, int E, int bin_rows, int64_t Tp_max,
                           int32_t* row_src, void* xp, bsg_stream_t stream);

/*
 * permute_pad_gate_backward - the backward's first step in one pass over
 * dy: what bsg_permute_pad(dy, ..., scale = gate, ...) writes (dyp, row_src)
 * and what bsg_route_backward writes (dlogits), the dot products
 * <dy_t, yp_j> taken while dy's rows are read for the permutation
 * (section 1.4's fused permutation kernel, here with the gate's gradient,
 * plain calculus on the gate of bsg_route).  Arguments as in those two
 * calls: dy [T, d] (dtype), gate [T*k] fp32 (the scale), yp [Tp_max, ld_yp]
 * (yp_dtype) the forward's expert outputs, logits [T, E] fp32, dlogits
 * [T, E] fp32 out.  fp32 dy needs fp32 yp (else BSG_EUNSUPPORTED).
 */
bsg_status bsg_permute_pad_gate_backward(const void* dy, int dtype, int64_t T, int d, int k,
                                         const int32_t* dest_row, const float* gate,
                                         const int32_t* counts, const int32_t* bin_offsets, int E,
                                         int bin_rows, int64_t Tp_max, int32_t* row_src,
                                         void* dyp, const float* logits, int renorm,
                                         const int32_t* expert_idx, const void* yp, int yp_dtype,
                                         int64_t ld_yp, float* dlogits, bsg_stream_t stream);

/*
 * build_topology - the topology + transpose metadata in ONE launch
 * (section 1.4, last paragraph): maps each expert's token row range to its
 * nonzero blocks.  Fills every array of *topo (see bsg_topology) from
 * bin_offsets [E+1]; f is the per-expert hidden width (multiple of 128).
 * topo->E, topo->F = f/128 and topo->Tp_max must match the arguments;
 * topo->block_rows is 128 or 64, and every bin offset must be a multiple of
 * it (else meta's status is 2 and the topology is published empty).
 */
bsg_status bsg_build_topology(const int32_t* bin_offsets, int E, int f, int64_t Tp_max,
                              const bsg_topology* topo /* host struct */, bsg_stream_t stream);

/*
 * route_topology - bsg_route followed by bsg_build_topology(bin_offsets, E,
 * f, Tp_max, topo), with the topology written by the routing's own
 * placement launch (section 1.4: the routing forms the bins, and the
 * topology with its transpose metadata follows from them alone).  Every
 * output, bit for bit, and every argument rule and error are those of the
 * two calls; two launches in all for routings of at most 65536 tokens whose
 * ceil(T/64) * E per-chunk counts number at most 65536, three above that.
 */
bsg_status bsg_route_topology(const float* logits, int64_t T, int E, int k, int renorm,
                              int bin_rows, int32_t* expert_idx, float* gate, int32_t* dest_row,
                              int32_t* counts, int32_t* bin_offsets, void* workspace,
                              size_t workspace_bytes, int f, int64_t Tp_max,
                              const bsg_topology* topo /* host struct */, bsg_stream_t stream);

/*
 * route_permute_topology - the forward's front in two launches (section 1.4:
 * route, then the fused gather + pad permutation, then the topology):
 * bsg_route, then bsg_permute_pad(x, dtype, T, d, k, dest_row, NULL,
 * counts, bin_offsets, E, bin_rows, Tp_max, row_src, xp), then, when topo
 * is not NULL, bsg_build_topology(bin_offsets, E, f, Tp_max, topo).  The
 * routing's placement launch also copies each token's row to its k places
 * (read once, written k times), zero-fills the pad rows and writes row_src.
 * Every output, bit for bit, and every argument rule and error are those of
 * the three calls (f is read only with a topology).  Two launches for
 * routings whose placement can sum the per-chunk counts itself, three
 * above that.
 */
bsg_status bsg_route_permute_topology(const float* logits, int64_t T, int E, int k, int renorm,
                                      int bin_rows, int32_t* expert_idx, float* gate,
                                      int32_t* dest_row, int32_t* counts, int32_t* bin_offsets,
                                      void* workspace, size_t workspace_bytes, const void* x,
                                      int dtype, int d, int64_t Tp_max, int32_t* row_src,
                                      void* xp, int f, const bsg_topology* topo /* or NULL */,
                                      bsg_stream_t stream);

/*
 * sdd - sampled dense-dense product (section 1.2, first layer):
 * for every nonzero block b = (r, c):
 *   acc_b[m][n] = sum_k a[BR*r + m][k] * B[k][128c + n],  k < K,
 * where a is [Tp_max, K] row-major with leading dimension lda and
 *   trans_b = 0: B[k][n] = b[k*ldb + n]    (b is [K, E*f], e.g. W1)
 *   trans_b = 1: B[k][n] = b[n*ldb + k]    (b is [E*f, K], e.g. W2 for dgrad)
 * and the epilogue writes out_blocks[b] (block-major [nnz_max][BR][128]):
 *   NONE      acc
 *   GELU      gelu(acc); if aux_out != NULL also aux_out[b] = gelu'(acc), the
 *             derivative the backward needs (stored in dtype)
 *   SILU_MUL  silu(acc) * acc2 where acc2 uses b2 in place of b (SwiGLU);
 *             if aux_out != NULL it is a two-plane block array that also
 *             receives silu(acc) (plane 0) and acc2 * silu'(acc) (plane 1),
 *             the factors the backward needs (stored in dtype)
 *   GELU_BWD  acc * aux_in[b]  (aux_in = the derivative blocks saved by GELU)
 *   SILU_MUL_BWD  aux_in is the two-plane array saved by SILU_MUL and
 *             out_blocks a two-plane array: plane 0 = acc * aux_in plane 1
 *             (gradient of the gate projection, acc = dA), plane 1 =
 *             acc * aux_in plane 0 (gradient of the up projection)
 * K must be a positive multiple of 64 (bf16) or 32 (fp32).
 */
bsg_status bsg_sdd(const void* a, int64_t lda, const void* b, const void* b2, int64_t ldb,
                   int trans_b, int K, const bsg_topology* topo, int epilogue,
                   const void* aux_in, void* out_blocks, void* aux_out, int dtype,
                   bsg_stream_t stream);

/*
 * dsd - dense = sparse x dense (section 1.2, second layer; walks each block
 * row through the BCSR row pointer as section 1.3 describes):
 *   c[BR*r + m][n] = sum over blocks b of row r, sum_j blocks[b][m][j] *
 *                    B[128*col_idx[b] + j][n],  n < N,
 *   trans_b = 0: B[k][n] = b[k*ldb + n]  (b is [E*f, N], e.g. W2)
 *   trans_b = 1: B[k][n] = b[n*ldb + k]  (b is [N, E*f], e.g. W1 for dgrad)
 * With blocks2 and b2 (both or neither; same topology, ldb and trans_b) the
 * sum also runs over blocks2[b] against B2 taken from b2 (SwiGLU input
 * gradient: gate projection with W1 plus up projection with W3), in one
 * fp32 accumulation.
 * c is [Tp_max, N] with leading dimension ldc in c_dtype (bf16 or fp32);
 * rows >= Tp are untouched.  N must be a positive multiple of 128.
 *
 * workspace (optional, NULL for none; caller-owned device memory, 256-byte
 * aligned, workspace_bytes >= 2 * BSG_DSD_SHARE_BYTES) lets the product split
 * its last, partly filled round of 256 x 256 tiles: when the tiles do not
 * fill whole rounds of the GPU's compute units, each of the last round's
 * tiles is cut into 2 to 8 K-segments whose fp32 partial sums (one share of
 * BSG_DSD_SHARE_BYTES each) go to the workspace, and a second launch adds
 * them in segment order and stores the tile.  Deterministic; the split
 * tiles' sums associate differently from an unsplit run (fp32 rounding).
 * Used only when a tile walks at least 32 K-blocks (f >= 4096, or the two
 * block sets together); otherwise, or with fewer shares than needed, the
 * workspace is ignored.  bsg_dsd_workspace_bytes gives the size that allows
 * every split.  Calls sharing one workspace must not overlap in time.
 */
bsg_status bsg_dsd(const void* blocks, const void* blocks2, const bsg_topology* topo,
                   const void* b, const void* b2, int64_t ldb, int trans_b, int N, void* c,
                   int64_t ldc, int c_dtype, int dtype, void* workspace, size_t workspace_bytes,
                   bsg_stream_t stream);

/* One share of bsg_dsd's workspace: the fp32 partial sums of a 256 x 256 tile. */
#define BSG_DSD_SHARE_BYTES 262144

/*
 * dsd_workspace_bytes - the bsg_dsd workspace that lets every split of its
 * last round happen on the device of `stream` (the current device for the
 * null stream): one share per compute unit.  A host-side size helper the
 * post does not define; it queries the device once (HIP errors reported as
 * BSG_EHIP).
 */
bsg_status bsg_dsd_workspace_bytes(bsg_stream_t stream, int64_t* bytes);

/*
 * dsd_combine_top1 - bsg_dsd followed by bsg_unpermute_combine for top-1
 * routing, in one launch: the product's rows leave the epilogue both to c
 * (as bsg_dsd writes it; c may be NULL when only y is wanted) and straight
 * to token order,
 *   y[row_src[r]][n] = rd(gate[row_src[r]] * rd(C[r][n]))  (gate NULL: 1)
 * for every row r below Tp with row_src[r] >= 0, which equals what
 * bsg_unpermute_combine(c, ..., k = 1, ...) writes, bit for bit (the
 * second layer and the reverse layout transform of section 1.4).  row_src
 * comes from bsg_permute_pad of a top-1 routing (assignment id = token).
 * bf16 only (blocks, b, c and y); y is [T, ldy].  One block set.
 */
bsg_status bsg_dsd_combine_top1(const void* blocks, const bsg_topology* topo, const void* b,
                                int64_t ldb, int trans_b, int N, void* c, int64_t ldc,
                                const int32_t* row_src, const float* gate, void* y, int64_t ldy,
                                int dtype, bsg_stream_t stream);

/*
 * dstd - dense = sparse^T x dense, the weight gradient (section 1.3,
 * "transpose indices": the blocks of each column are those trans_idx lists,
 * their rows those row_idx gives; the kernel computes both from col_ptr):
 *   C[128c + m][n] = sum over blocks b of column c, sum_j blocks[b][j][m] *
 *                    dmat[BR*row_idx[b] + j][n],  n < N
 * dmat is [Tp_max, N] with leading dimension ldd.  trans_c = 0 stores
 * C at c[(128c + m)*ldc + n] ([E*f, N], e.g. dW2); trans_c = 1 stores it
 * transposed at c[n*ldc + 128c + m] ([N, E*f], e.g. dW1).  Columns with no
 * block (experts without tokens) are written as zeros.  N must be a
 * positive multiple of 128.  The output dtype is dtype.
 */
bsg_status bsg_dstd(const void* blocks, const bsg_topology* topo, const void* dmat, int64_t ldd,
                     int N, void* c, int64_t ldc, int trans_c, int dtype, bsg_stream_t stream);

/*
 * unpermute_combine - undo the permutation and combine the k expert
 * outputs of each token (the inverse of the layout transform of
 * section 1.4):  y[t][m] = sum_{j<k} gate[t*k+j] * yp[dest_row[t*k+j]][m],
 * accumulated in fp32 in ascending j and rounded once to y_dtype;
 * gate == NULL means every gate is 1 (input-gradient combine).
 *   yp [Tp_max, d] (yp_dtype, leading dimension ld_yp), y [T, d] (y_dtype);
 *   every dest_row entry must be below yp's Tp_max (it is when yp was sized
 *   with bsg_max_padded_rows for the bin size the routing used).
 */
bsg_status bsg_unpermute_combine(const void* yp, int yp_dtype, int64_t ld_yp,
                                 const int32_t* dest_row, const float* gate, int64_t T, int k,
                                 int d, void* y, int y_dtype, bsg_stream_t stream);

/*
 * stream_copy - a plain device-to-device copy of `bytes` bytes (a multiple of
 * 16; src and dst 16-byte aligned, not overlapping), every byte read once
 * and written once.  Not a step of the method: the HBM ceiling that the
 * data-movement calls (permute_pad, unpermute_combine) are measured against,
 * and a way to write enough memory to evict the last-level cache between
 * timed runs.
 */
bsg_status bsg_stream_copy(const void* src, void* dst, size_t bytes, bsg_stream_t stream);

/* Static description of a status code. */
const char* bsg_status_string(bsg_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* bsg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
