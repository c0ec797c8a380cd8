// split_g4.hip -- the split-pass kernels for GQA groups of 4 query heads
// (contiguous and paged rows, every stored row width).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g4(const SplitArgs &a, hipStream_t s)
{
    return a.geom.bs > 0 ? launch_split_g<4, true>(a, s) : launch_split_g<4, false>(a, s);
}

} // namespace swan
