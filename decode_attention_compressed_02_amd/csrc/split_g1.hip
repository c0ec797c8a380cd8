// split_g1.hip -- the split-pass kernels for GQA groups of 1 query head
// (contiguous and paged rows, every stored row width).
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g1(const SplitArgs &a, hipStream_t s)
{
    return a.geom.bs > 0 ? launch_split_g<1, true>(a, s) : launch_split_g<1, false>(a, s);
}

} // namespace swan
