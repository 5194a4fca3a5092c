// The block-sparse products for blocks of 64 rows: the finer bins of the
// block-size study (George Lin's Blog, MegaBlocks post, section 1.3, block
// size), whose 64-row bins cannot share a 128-row block.
#include "gemm.hpp"

namespace bsg {
BSG_GEMM_INSTANTIATE(64)
}  // namespace bsg
