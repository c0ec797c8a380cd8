// split_g1_paged.hip -- the split-pass kernels for GQA groups of 1 query
// head over a paged pool (rows through the block table).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g1_paged(const SplitArgs &a, hipStream_t s) { return launch_split_g<1, true>(a, s); }

} // namespace swan
