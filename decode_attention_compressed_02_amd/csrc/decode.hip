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

__device__ __forceinline__ int64_t block_sum128(int64_t v, int64_t *red)
{
    const int t = threadIdx.x;
    v = lane_value(wave_scan(v), kWave - 1);
    if ((t & (kWave - 1)) == 0) red[t / kWave] = v;
    __syncthreads();
    v = red[0] + red[1];
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(128) void k_reduce(ReduceArgs a)
{
    __shared__ float wsh[128];
    __shared__ float redf[2];
    __shared__ int64_t red[2];
    const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int G = a.N_h / a.H, h = hq / G, hh = hq % G;
    float *out = a.o_hat + ((int64_t)b * a.N_h + hq) * kD + t;

    int64_t tot = 0, before = 0;
    for (int bb = t; bb < a.B; bb += 128) {
        const int64_t len = seq_work(a.pos, bb, a.R, a.row_cap, a.row_bytes);
        tot += len;
        if (bb < b) before += len;
    }
    tot = block_sum128(tot, red);
    before = block_sum128(before, red);
    const int64_t len = unit_work(a.pos[b], a.R, a.row_cap, a.row_bytes).len;
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

    float mx = -INFINITY;
    for (int64_t w = w0 + t; w <= w1; w += 128) mx = fmaxf(mx, ml[w * ml_step]);
    mx = wave_max(mx);
    if ((t & (kWave - 1)) == 0) redf[t / kWave] = mx;
    __syncthreads();
    mx = fmaxf(redf[0], redf[1]);
    __syncthreads();

    float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    for (int64_t c0 = w0; c0 <= w1; c0 += 128) {
        const int64_t w = c0 + t;
        float wt = 0.f;
        if (w <= w1) {
            wt = exp2f(ml[w * ml_step] - mx);
            L = fmaf(wt, ml[w * ml_step + 1], L);
        }
        wsh[t] = wt;
        __syncthreads();
        const int cnt = (int)min((int64_t)128, w1 - c0 + 1);
        const float *pc = po + c0 * po_step;
        int j = 0;
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
    if ((t & (kWave - 1)) == 0) redf[t / kWave] = L;
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
