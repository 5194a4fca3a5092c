/*
 * A C caller of the library: the dropless-MoE layer's forward through the C
 * ABI alone (include/bsg.h), every device buffer from hipMalloc, no Python
 * or torch.  The calls follow the forward of George Lin's Blog
 * (MegaBlocks/FlexMoE post, sections 1.2-1.4): route, permute_pad,
 * build_topology, sdd with GeLU, dsd, unpermute_combine.
 *
 * Usage: bsg_forward_demo <dir> T d E f k
 * reads <dir>/logits.f32 [T, E], <dir>/x.bf16 [T, d], <dir>/w1.bf16
 * [d, E*f], <dir>/w2.bf16 [E*f, d] (raw little-endian arrays) and writes
 * <dir>/y.bf16 [T, d].  It also checks that an invalid call is refused
 * with BSG_EINVAL before any launch.  Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsg.h"

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
            return 1;                                                             \
        }                                                                         \
    } while (0)

#define BSG_OK_(call)                                                             \
    do {                                                                          \
        bsg_status s_ = (call);                                                   \
        if (s_ != BSG_OK) {                                                       \
            fprintf(stderr, "%s: %s (%s)\n", #call, bsg_status_string(s_),        \
                    bsg_last_error());                                            \
            return 1;                                                             \
        }                                                                         \
    } while (0)

static int read_file(const char* dir, const char* name, void* dst, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        return 1;
    }
    size_t got = fread(dst, 1, bytes, f);
    fclose(f);
    if (got != bytes) {
        fprintf(stderr, "%s: %zu of %zu bytes\n", path, got, bytes);
        return 1;
    }
    return 0;
}

static int upload(const char* dir, const char* name, void** dev, size_t bytes) {
    void* host = malloc(bytes);
    if (!host || read_file(dir, name, host, bytes)) {
        free(host);
        return 1;
    }
    hipError_t e = hipMalloc(dev, bytes);
    if (e == hipSuccess) e = hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice);
    free(host);
    if (e != hipSuccess) {
        fprintf(stderr, "upload %s: %s\n", name, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 7) {
        fprintf(stderr, "usage: %s <dir> T d E f k\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    const int64_t T = atoll(argv[2]);
    const int d = atoi(argv[3]), E = atoi(argv[4]), f = atoi(argv[5]), k = atoi(argv[6]);
    const int bin_rows = BSG_BLOCK;

    /* capacities: every routing-dependent size from the host size queries */
    const int64_t Tp_max = bsg_max_padded_rows(T, k, E, bin_rows);
    bsg_topo_sizes sz;
    if (Tp_max < 0) {
        fprintf(stderr, "bad sizes\n");
        return 2;
    }
    BSG_OK_(bsg_topology_sizes(Tp_max, E, f, BSG_BLOCK, &sz));
    const size_t ws_bytes = bsg_route_workspace_bytes(T, k, E);
    const int64_t A = T * k, ncol = (int64_t)E * f;

    void *logits, *x, *w1, *w2;
    if (upload(dir, "logits.f32", &logits, (size_t)T * E * 4) ||
        upload(dir, "x.bf16", &x, (size_t)T * d * 2) ||
        upload(dir, "w1.bf16", &w1, (size_t)d * ncol * 2) ||
        upload(dir, "w2.bf16", &w2, (size_t)ncol * d * 2))
        return 1;

    int32_t *expert_idx, *dest_row, *counts, *bin_offsets, *row_src;
    float* gate;
    void *ws, *xp, *act, *yp, *y;
    HIP_OK(hipMalloc((void**)&expert_idx, (size_t)A * 4));
    HIP_OK(hipMalloc((void**)&gate, (size_t)A * 4));
    HIP_OK(hipMalloc((void**)&dest_row, (size_t)A * 4));
    HIP_OK(hipMalloc((void**)&counts, (size_t)E * 4));
    HIP_OK(hipMalloc((void**)&bin_offsets, (size_t)(E + 1) * 4));
    HIP_OK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 16));
    HIP_OK(hipMalloc((void**)&row_src, (size_t)Tp_max * 4));
    HIP_OK(hipMalloc(&xp, (size_t)Tp_max * d * 2));
    HIP_OK(hipMalloc(&act, (size_t)sz.nnz_max * BSG_BLOCK * BSG_BLOCK * 2));
    HIP_OK(hipMalloc(&yp, (size_t)Tp_max * d * 2));
    HIP_OK(hipMalloc(&y, (size_t)T * d * 2));

    bsg_topology topo;
    memset(&topo, 0, sizeof topo);
    HIP_OK(hipMalloc((void**)&topo.row_ptr, (size_t)(sz.row_blocks_max + 1) * 4));
    HIP_OK(hipMalloc((void**)&topo.col_idx, (size_t)sz.nnz_max * 4));
    HIP_OK(hipMalloc((void**)&topo.row_idx, (size_t)sz.nnz_max * 4));
    HIP_OK(hipMalloc((void**)&topo.col_ptr, (size_t)(sz.n_cols + 1) * 4));
    HIP_OK(hipMalloc((void**)&topo.trans_idx, (size_t)sz.nnz_max * 4));
    HIP_OK(hipMalloc((void**)&topo.row_tiles, (size_t)sz.row_tiles_max * 4));
    HIP_OK(hipMalloc((void**)&topo.expert_order, (size_t)E * 4));
    HIP_OK(hipMalloc((void**)&topo.meta, 4 * 4));
    topo.E = E;
    topo.F = f / BSG_BLOCK;
    topo.block_rows = BSG_BLOCK;
    topo.Tp_max = Tp_max;

    /* an invalid call is refused before any launch (K not a multiple of 64) */
    if (bsg_sdd(xp, d, w1, NULL, ncol, 0, 100, &topo, BSG_EPI_GELU, NULL, act, NULL, BSG_BF16,
                NULL) != BSG_EINVAL) {
        fprintf(stderr, "an invalid sdd call was not refused\n");
        return 1;
    }

    /* the forward, all on the null stream */
    BSG_OK_(bsg_route((const float*)logits, T, E, k, 0, bin_rows, expert_idx, gate, dest_row,
                      counts, bin_offsets, ws, ws_bytes, NULL));
    BSG_OK_(bsg_permute_pad(x, BSG_BF16, T, d, k, dest_row, NULL, counts, bin_offsets, E,
                            bin_rows, Tp_max, row_src, xp, NULL));
    BSG_OK_(bsg_build_topology(bin_offsets, E, f, Tp_max, &topo, NULL));
    BSG_OK_(bsg_sdd(xp, d, w1, NULL, ncol, 0, d, &topo, BSG_EPI_GELU, NULL, act, NULL, BSG_BF16,
                    NULL));
    BSG_OK_(bsg_dsd(act, NULL, &topo, w2, NULL, d, 0, d, yp, d, BSG_BF16, BSG_BF16, NULL, 0, NULL));
    BSG_OK_(bsg_unpermute_combine(yp, BSG_BF16, d, dest_row, gate, T, k, d, y, BSG_BF16, NULL));
    HIP_OK(hipDeviceSynchronize());

    size_t ybytes = (size_t)T * d * 2;
    void* host = malloc(ybytes);
    if (!host) return 1;
    HIP_OK(hipMemcpy(host, y, ybytes, hipMemcpyDeviceToHost));
    char path[4096];
    snprintf(path, sizeof path, "%s/y.bf16", dir);
    FILE* out = fopen(path, "wb");
    if (!out || fwrite(host, 1, ybytes, out) != ybytes) {
        fprintf(stderr, "cannot write %s\n", path);
        return 1;
    }
    fclose(out);
    free(host);
    printf("forward ok: T=%lld d=%d E=%d f=%d k=%d Tp_max=%lld\n", (long long)T, d, E, f, k,
           (long long)Tp_max);
    return 0;
}
