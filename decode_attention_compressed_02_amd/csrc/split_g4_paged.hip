// split_g4_paged.hip -- the split-pass kernels for GQA groups of 4 query
// heads over a paged pool (rows through the block table).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g4_paged(const SplitArgs &a, hipStream_t s) { return launch_split_g<4, true>(a, s); }

} // namespace swan
