// decode.hip -- pass 2 of the hybrid decode attention (the merge of the split
// pass's partials) and the dispatch of the split pass, whose kernel lives in
// split_kernel.h and is instantiated per GQA group size in split_g*.hip (so
// that the instantiations compile in parallel).
#include "split_kernel.h"

namespace swan {

// ---------------------------------------------------------------------------
// pass 2: merge the partials of one (query head, sequence): the pieces of its
// unit, found from the same work plan as the split pass.  Thread c owns
// output coordinate c.  A unit with no tokens (inactive sequence) yields zeros.
// ---------------------------------------------------------------------------

// pieces whose output coordinate a thread loads together with the (m, l)
// pairs, before the max is known: a unit of up to this many pieces costs one
// round trip to memory after the work plan, not three
constexpr int kReducePrefetch = 16;

__global__ __launch_bounds__(128) void k_reduce(ReduceArgs a)
{
    __shared__ float wsh[128];
    __shared__ float redf[2];
    __shared__ int64_t red[2][2];
    const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x, wv = t / kWave;
    const int G = a.N_h / a.H, h = hq / G, hh = hq % G;
    float *out = a.o_hat + ((int64_t)b * a.N_h + hq) * kD + t;

    // work rows of the whole batch and of the sequences before b
    const int32_t pb = a.pos[b];
    int64_t tot = 0, before = 0;
    for (int bb = t; bb < a.B; bb += 128) {
        const int64_t len = seq_work(a.pos, bb, a.R, a.row_cap, a.row_bytes);
        tot += len;
        if (bb < b) before += len;
    }
    tot = lane_value(wave_scan(tot), kWave - 1);
    before = lane_value(wave_scan(before), kWave - 1);
    if ((t & (kWave - 1)) == 0) {
        red[wv][0] = tot;
        red[wv][1] = before;
    }
    __syncthreads();
    tot = red[0][0] + red[1][0];
    before = red[0][1] + red[1][1];
    const int64_t len = unit_work(pb, a.R, a.row_cap, a.row_bytes).len;
    if (len == 0) {
        *out = 0.f;
        return;
    }
    // waves whose ranges [w T / V, (w + 1) T / V) meet [us, us + len)
    const int64_t T = tot * a.H, V = active_waves(T, a.W, a.split_tokens);
    const int64_t us = before * a.H + h * len, u = (int64_t)b * a.H + h;
    const int64_t w0 = max(((us + 1) * V + T - 1) / T - 1, (int64_t)0);
    const int64_t w1 = min(((us + len) * V + T - 1) / T - 1, V - 1);
    // partial of wave w: index w + u, head hh
    const float *ml = a.part_ml + (u * G + hh) * 2;
    const float *po = a.part_o + (u * G + hh) * kD + t;
    const int64_t ml_step = (int64_t)G * 2, po_step = (int64_t)G * kD;

    // the first chunk's (m, l) and the first pieces' outputs, all in flight at once
    f32x2 ml0 = {-INFINITY, 0.f};
    if (w0 + t <= w1) ml0 = *(const f32x2 *)(ml + (w0 + t) * ml_step);
    float pre[kReducePrefetch];
#pragma unroll
    for (int j = 0; j < kReducePrefetch; ++j) pre[j] = w0 + j <= w1 ? po[(w0 + j) * po_step] : 0.f;

    float mx = ml0.x;
    for (int64_t w = w0 + 128 + t; w <= w1; w += 128) mx = fmaxf(mx, ml[w * ml_step]);
    mx = wave_max(mx);
    if ((t & (kWave - 1)) == 0) redf[wv] = mx;
    __syncthreads();
    mx = fmaxf(redf[0], redf[1]);
    __syncthreads();

    float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    for (int64_t c0 = w0; c0 <= w1; c0 += 128) {
        const int64_t w = c0 + t;
        float wt = 0.f;
        if (w <= w1) {
            const f32x2 v = c0 == w0 ? ml0 : *(const f32x2 *)(ml + w * ml_step);
            wt = exp2f(v.x - mx);
            L = fmaf(wt, v.y, L);
        }
        wsh[t] = wt; // 0 past the last piece
        __syncthreads();
        const int cnt = (int)min((int64_t)128, w1 - c0 + 1);
        const float *pc = po + c0 * po_step;
        int j = 0;
        if (c0 == w0) {
#pragma unroll
            for (int jj = 0; jj < kReducePrefetch; jj += 4) {
                o0 = fmaf(wsh[jj], pre[jj], o0);
                o1 = fmaf(wsh[jj + 1], pre[jj + 1], o1);
                o2 = fmaf(wsh[jj + 2], pre[jj + 2], o2);
                o3 = fmaf(wsh[jj + 3], pre[jj + 3], o3);
            }
            j = kReducePrefetch;
        }
        for (; j + 4 <= cnt; j += 4) {
            o0 = fmaf(wsh[j], pc[j * po_step], o0);
            o1 = fmaf(wsh[j + 1], pc[(j + 1) * po_step], o1);
            o2 = fmaf(wsh[j + 2], pc[(j + 2) * po_step], o2);
            o3 = fmaf(wsh[j + 3], pc[(j + 3) * po_step], o3);
        }
        for (; j < cnt; ++j) o0 = fmaf(wsh[j], pc[j * po_step], o0);
        __syncthreads();
    }
    L = wave_sum(L);
    if ((t & (kWave - 1)) == 0) redf[wv] = L;
    __syncthreads();
    L = redf[0] + redf[1];
    const float o = (o0 + o1) + (o2 + o3);
    *out = L > 0.f ? o / L : 0.f;
}

hipError_t launch_split(const SplitArgs &a, int g, hipStream_t s)
{
    switch (g) {
    case 1: return launch_split_g1(a, s);
    case 2: return launch_split_g2(a, s);
    case 4: return launch_split_g4(a, s);
    case 8: return launch_split_g8(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_reduce, dim3(a.N_h, a.B), dim3(kD), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
