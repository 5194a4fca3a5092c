// The block-sparse products for blocks of 128 rows (the block of George
// Lin's Blog's MegaBlocks post, section 1.3).
#include "gemm.hpp"

namespace bsg {
BSG_GEMM_INSTANTIATE(128)
}  // namespace bsg
