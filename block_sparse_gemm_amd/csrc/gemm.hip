// Entry points of the block-sparse products (SDD, DSD, DSTD): the kernels
// live in gemm.hpp, instantiated per block height (gemm_br128.hip,
// gemm_br64.hip); the topology's block height picks the instantiation.
#include "kernels.hpp"

namespace bsg {

template <int BR>
hipError_t launch_sdd_br(const GemmParams& p, int64_t row_tiles_max, int trans_b, int epi,
                         int dtype, hipStream_t s);
template <int BR>
hipError_t launch_dsd_br(const GemmParams& p, int64_t row_tiles_max, int trans_b, int c_dtype,
                         int dtype, hipStream_t s);
template <int BR>
hipError_t launch_dstd_br(const GemmParams& p, int trans_c, int dtype, hipStream_t s);

hipError_t launch_sdd(const GemmParams& p, int64_t row_tiles_max, int trans_b, int epi, int dtype,
                      hipStream_t s) {
    return p.br == 64 ? launch_sdd_br<64>(p, row_tiles_max, trans_b, epi, dtype, s)
                      : launch_sdd_br<128>(p, row_tiles_max, trans_b, epi, dtype, s);
}

hipError_t launch_dsd(const GemmParams& p, int64_t row_tiles_max, int trans_b, int c_dtype,
                      int dtype, hipStream_t s) {
    return p.br == 64 ? launch_dsd_br<64>(p, row_tiles_max, trans_b, c_dtype, dtype, s)
                      : launch_dsd_br<128>(p, row_tiles_max, trans_b, c_dtype, dtype, s);
}

hipError_t launch_dstd(const GemmParams& p, int trans_c, int dtype, hipStream_t s) {
    return p.br == 64 ? launch_dstd_br<64>(p, trans_c, dtype, s)
                      : launch_dstd_br<128>(p, trans_c, dtype, s);
}

}  // namespace bsg
