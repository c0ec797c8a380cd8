// append.hip -- put the new token in the dense buffer; the token leaving the
// buffer is pruned to its k largest-magnitude coordinates and appended to
// the sparse history (SWAN page, hybrid-cache and pruning paragraphs).  The
// buffer is circular with slot = position mod R ("Reuse, Evict, or Limit
// Earlier Context", section 3.2), so the evicted token is exactly the one
// in the new token's slot.
//
// One workgroup of two waves per (kv head, sequence): wave 0 handles the
// key, wave 1 the value.  Each lane owns coordinates lane and lane + 64.
#include "swan_internal.h"

namespace swan {

__global__ __launch_bounds__(128) void k_append(AppendArgs a)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t u = (int64_t)b * a.H + h;
    uint16_t lo, hi;
    if (wave == 0) {
        lo = a.k_hat[u * kD + lane];
        hi = a.k_hat[u * kD + lane + 64];
    } else {
        lo = f2h(a.v_hat[u * kD + lane]);
        hi = f2h(a.v_hat[u * kD + lane + 64]);
    }
    append_token(a, b, h, wave, lane, lo, hi);
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_append, dim3(a.H, a.B), dim3(128), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
