// split_g1_paged.hip -- the split-pass kernels for GQA groups of 1 query head over
// a paged pool whose ring slots each lie in one block (one block id per
// slot); other block sizes use split_g1_paged_rows.hip.
#include "split_kernel.h"

namespace swan {

hipError_t launch_split_g1_paged(const SplitArgs &a, hipStream_t s)
{
    return paged_slot_blocks(1, a.geom) ? launch_split_g<1, true, true>(a, s) : launch_split_g1_paged_rows(a, s);
}

} // namespace swan
