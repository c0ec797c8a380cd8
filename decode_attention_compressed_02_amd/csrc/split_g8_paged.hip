// split_g8_paged.hip -- the split-pass kernels for GQA groups of 8 query heads over
// a paged pool whose ring slots each lie in one block (one block id per
// slot); other block sizes use split_g8_paged_rows.hip.
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g8_paged(const SplitArgs &a, hipStream_t s)
{
    return paged_slot_blocks(8, a.geom) ? launch_split_g<8, true, true>(a, s) : launch_split_g8_paged_rows(a, s);
}

} // namespace swan
