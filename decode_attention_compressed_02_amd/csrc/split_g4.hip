// split_g4.hip -- the split-pass kernels for GQA groups of 4 query heads,
// contiguous rows, every pair of stored key and value row widths; paged rows
// are instantiated in split_g4_paged.hip so the two compile in parallel.
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g4(const SplitArgs &a, hipStream_t s)
{
    return a.geom.bs > 0 ? launch_split_g4_paged(a, s) : launch_split_g<4, false>(a, s);
}

} // namespace swan
