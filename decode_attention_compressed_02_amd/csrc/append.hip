// append.hip -- put the new token in the dense buffer; the token leaving the
// buffer is pruned to its k largest-magnitude coordinates and appended to
// the sparse history (SWAN section 4.2, hybrid cache and pruning).  The
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
    const int p = a.pos[b];
    if (p < 0) return;

    const int64_t u = (int64_t)b * a.H + h;
    uint16_t nlo, nhi;
    if (wave == 0) {
        nlo = a.k_hat[u * kD + lane];
        nhi = a.k_hat[u * kD + lane + 64];
    } else {
        nlo = f2h(a.v_hat[u * kD + lane]);
        nhi = f2h(a.v_hat[u * kD + lane + 64]);
    }
    uint8_t *idx = wave == 0 ? a.kidx : a.vidx;
    uint16_t *val = wave == 0 ? a.kval : a.vval;
    const int row_cap = a.geom.bs > 0 ? a.geom.max_blocks * a.geom.bs : a.geom.n_cap;

    if (a.R == 0) {
        // no buffer: the new token is pruned straight into sparse row p
        const int64_t off = p < row_cap ? row_offset_rt(a.geom, b, h, p) : -1;
        if (off >= 0) wave_prune_row(lane, nlo, nhi, a.k, a.geom.ks, idx + off, val + off);
        return;
    }
    uint16_t *buf = (wave == 0 ? a.kbuf : a.vbuf) + (u * a.R + p % a.R) * kD;
    if (p >= a.R) {
        // the slot holds token p - R, the oldest one: evict and prune it
        const uint16_t olo = buf[lane], ohi = buf[lane + 64];
        const int r = p - a.R;
        const int64_t off = r < row_cap ? row_offset_rt(a.geom, b, h, r) : -1;
        if (off >= 0) wave_prune_row(lane, olo, ohi, a.k, a.geom.ks, idx + off, val + off);
    }
    buf[lane] = nlo;
    buf[lane + 64] = nhi;
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_append, dim3(a.H, a.B), dim3(128), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
