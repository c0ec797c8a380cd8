// split_g8_paged_rows.hip -- the split-pass kernels for GQA groups of 8
// query heads over a paged pool whose block size is not a power-of-two
// multiple of the ring-slot rows: rows looked up one at a time.
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g8_paged_rows(const SplitArgs &a, hipStream_t s) { return launch_split_g<8, true, false>(a, s); }

} // namespace swan
