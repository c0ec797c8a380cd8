// split_g2.hip -- the split-pass kernels for GQA groups of 2 query heads
// (contiguous and paged rows, every stored row width).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g2(const SplitArgs &a, hipStream_t s)
{
    return a.geom.bs > 0 ? launch_split_g<2, true>(a, s) : launch_split_g<2, false>(a, s);
}

} // namespace swan
