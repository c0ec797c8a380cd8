// prefill.hip -- convert a prefilled history into the hybrid cache (the step
// before decoding starts: the SWAN page's hybrid cache keeps the newest R tokens dense
// and every older one as its pruned sparse row).
//
// One workgroup of 256 threads per (32-token tile, kv head, sequence):
//   1. RoPE of the tile's raw keys at their own positions into LDS,
//      transposed as xs[c][token];
//   2. the tile times P_QK (thread = output column j and a 16-token half),
//      rounded once to fp16; values rounded to fp16;
//   3. each wave places 8 tokens: tokens older than len - R are pruned into
//      their sparse rows (the same wave-level top-k as the append kernel),
//      the newest R go to buffer slots t mod R.
// The result is identical to appending the tokens one at a time.  Keys are
// rotated and projected in double, as in the decode-step projection, so that
// their fp16 rounding (and with it the pruning) does not depend on float
// rounding of intermediate products.
#include "swan_internal.h"

namespace swan {

constexpr int kTile = 32;

__global__ __launch_bounds__(256) void k_prefill(PrefillArgs a)
{
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = min(a.len[b], a.max_len);
    const int t0 = tile * kTile;
    if (t0 >= T) return;

    __shared__ __attribute__((aligned(16))) double xs[kD][kTile + 2];
    __shared__ uint16_t kh[kTile][kD], vh[kTile][kD];

    const int64_t u = (int64_t)b * a.H + h;
    const float *kr = a.k_raw + u * a.T_stride * kD;
    const float *vr = a.v_hat + u * a.T_stride * kD;
    for (int e = tid; e < kTile * (kD / 2); e += 256) {
        const int tt = e / (kD / 2), i = e % (kD / 2), t = t0 + tt;
        double y0 = 0.0, y1 = 0.0;
        if (t < T) {
            const double theta = pow((double)a.base, -(double)i / (double)(kD / 2));
            double sn, cs;
            sincos((double)t * theta, &sn, &cs);
            const double x0 = kr[(int64_t)t * kD + i], x1 = kr[(int64_t)t * kD + i + kD / 2];
            y0 = x0 * cs - x1 * sn;
            y1 = x1 * cs + x0 * sn;
        }
        xs[i][tt] = y0;
        xs[i + kD / 2][tt] = y1;
    }
    for (int e = tid; e < kTile * kD; e += 256) {
        const int tt = e / kD, c = e % kD, t = t0 + tt;
        vh[tt][c] = t < T ? f2h(vr[(int64_t)t * kD + c]) : (uint16_t)0;
    }
    __syncthreads();

    {
        const int j = tid % kD, half = tid / kD; // tokens half*16 .. half*16+15
        double acc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[q] = 0.0;
        const float *P = a.P + ((int64_t)(b / a.Bl) * a.H + h) * kD * kD + j;
        for (int c = 0; c < kD; ++c) {
            const double pc = P[c * kD];
            const double *xr = &xs[c][half * 16];
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[q] = fma(xr[q], pc, acc[q]);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) kh[half * 16 + q][j] = d2h(acc[q]);
    }
    __syncthreads();

    const int row_cap = a.geom.bs > 0 ? a.geom.max_blocks * a.geom.bs : a.geom.n_cap;
    for (int q = 0; q < kTile / 4; ++q) {
        const int tt = wave * (kTile / 4) + q, t = t0 + tt;
        if (t >= T) break; // wave-uniform
        for (int which = 0; which < 2; ++which) {
            const uint16_t lo = which ? vh[tt][lane] : kh[tt][lane];
            const uint16_t hi = which ? vh[tt][lane + 64] : kh[tt][lane + 64];
            if (t < T - a.R) {
                const int64_t slot = t < row_cap ? row_slot_rt(a.geom, b, h, t) : -1;
                const int kk = which ? a.k_v : a.k, ks = which ? a.geom.ks_v : a.geom.ks;
                if (slot >= 0)
                    wave_prune_row(lane, lo, hi, kk, ks, (which ? a.vidx : a.kidx) + slot * ks,
                                   (which ? a.vval : a.kval) + slot * ks * a.geom.vbytes, a.geom.vbytes);
            } else {
                uint16_t *buf = (which ? a.vbuf : a.kbuf) + (u * a.R + t % a.R) * kD;
                buf[lane] = lo;
                buf[lane + 64] = hi;
            }
        }
    }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s)
{
    const dim3 grid((a.max_len + kTile - 1) / kTile, a.H, a.B);
    hipLaunchKernelGGL(k_prefill, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
