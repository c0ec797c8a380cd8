// project.hip -- runtime projection of the new query and key (SWAN section
// 4.1: RoPE is position dependent, so RoPE(x) P_QK cannot be folded into the
// weights and runs every decode step).
//
// One workgroup per (kv head, sequence), 128 threads (thread j = output
// coordinate j).  The g query vectors of the GQA group and the new key are
// rotated by RoPE into LDS, then every thread walks the 128 rows of P_QK
// once (coalesced 512-byte rows, L2-resident across sequences) and applies
// each row to all g + 1 vectors.  The 4 d_h^2 FLOPs per head of SWAN
// appendix A.2 are tiny next to the decode stream, so plain FMA is used.
#include "swan_internal.h"

namespace swan {

template <int G>
__global__ __launch_bounds__(128) void k_project(ProjectArgs a)
{
    const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
    __shared__ float xs[G + 1][kD];
    __shared__ float cs[kD / 2], sn[kD / 2];

    const int p = max(a.pos[b], 0);
    if (j < kD / 2) {
        // angle in double: at positions ~1e5 a float angle is off by ~1e-2 rad
        const double theta = pow((double)a.base, -(double)j / (double)(kD / 2));
        double s, c;
        sincos((double)p * theta, &s, &c);
        cs[j] = (float)c;
        sn[j] = (float)s;
    }
    __syncthreads();
    // RoPE: pair (i, i + 64) rotated by angle_i; 128 threads cover 2 vectors per pass
    for (int v = j / (kD / 2); v < G + 1; v += 2) {
        const int i = j % (kD / 2);
        const float *x = (v < G) ? a.q + ((int64_t)b * a.N_h + h * G + v) * kD : a.k + ((int64_t)b * a.H + h) * kD;
        const float x0 = x[i], x1 = x[i + kD / 2];
        xs[v][i] = x0 * cs[i] - x1 * sn[i];
        xs[v][i + kD / 2] = x1 * cs[i] + x0 * sn[i];
    }
    __syncthreads();

    float acc[G + 1];
#pragma unroll
    for (int v = 0; v < G + 1; ++v) acc[v] = 0.f;
    const float *P = a.P + (int64_t)h * kD * kD + j;
#pragma unroll 4
    for (int c = 0; c < kD; ++c) {
        const float pc = P[c * kD];
#pragma unroll
        for (int v = 0; v < G + 1; ++v) acc[v] = fmaf(xs[v][c], pc, acc[v]);
    }
#pragma unroll
    for (int v = 0; v < G; ++v) a.q_hat[((int64_t)b * a.N_h + h * G + v) * kD + j] = acc[v];
    a.k_hat[((int64_t)b * a.H + h) * kD + j] = f2h(acc[G]);
}

hipError_t launch_project(const ProjectArgs &a, hipStream_t s)
{
    const dim3 grid(a.H, a.B);
    switch (a.N_h / a.H) {
    case 1: hipLaunchKernelGGL(k_project<1>, grid, dim3(128), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_project<2>, grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_project<4>, grid, dim3(128), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_project<8>, grid, dim3(128), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace swan
