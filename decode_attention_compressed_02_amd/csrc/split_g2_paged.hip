// split_g2_paged.hip -- the split-pass kernels for GQA groups of 2 query heads over
// a paged pool whose ring slots each lie in one block (one block id per
// slot); other block sizes use split_g2_paged_rows.hip.
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g2_paged(const SplitArgs &a, hipStream_t s)
{
    return paged_slot_blocks(2, a.geom) ? launch_split_g<2, true, true>(a, s) : launch_split_g2_paged_rows(a, s);
}

} // namespace swan
