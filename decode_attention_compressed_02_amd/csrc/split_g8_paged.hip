// split_g8_paged.hip -- the split-pass kernels for GQA groups of 8 query
// heads over a paged pool (rows through the block table).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g8_paged(const SplitArgs &a, hipStream_t s) { return launch_split_g<8, true>(a, s); }

} // namespace swan
