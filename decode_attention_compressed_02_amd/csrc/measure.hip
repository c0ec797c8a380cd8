// measure.hip -- the yardsticks of swan_measure.h: how fast this GPU reads a
// buffer once from HBM (the ceiling for a decode step that must read its
// whole cache every step), and how fast its matrix cores run fp64 products
// (the ceiling for the prefill conversion's double-precision projection).
//
// One-wave workgroups each read one contiguous share of the buffer with
// 16-byte non-temporal loads (lane l takes every 64th 16-byte unit from
// l), eight loads in flight a lane, and fold the words into one register
// that is stored at the end, so no load can be dropped.
#include "swan_internal.h"

namespace swan {

typedef uint32_t msr_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void k_stream_read(const msr_u32x4 *p, int64_t n16, uint32_t *sink)
{
    constexpr int kInFlight = 8;
    const int lane = threadIdx.x;
    const int64_t w = blockIdx.x, W = gridDim.x;
    const int64_t lo = w * n16 / W, hi = (w + 1) * n16 / W;
    uint32_t acc = 0;
    int64_t i = lo + lane;
    for (; i + (kInFlight - 1) * kWave < hi; i += kInFlight * kWave) {
        msr_u32x4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) v[j] = __builtin_nontemporal_load(p + i + j * kWave);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < hi; i += kWave) {
        const msr_u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[w * kWave + lane] = acc;
}

hipError_t launch_stream_read(const void *buf, int64_t bytes, int waves, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(k_stream_read, dim3(waves), dim3(kWave), 0, s, (const msr_u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

// fp64 matrix-core rate: every wave runs `iters` rounds of eight independent
// 16x16x4 products (A and B all x), so each accumulator element gains 4 x^2
// a round; the lane's four elements of all eight accumulators are summed
// into sink[wave * 64 + lane] (128 x^2 iters when exact).  Workgroups of
// four waves (one per SIMD of a CU); waves past `waves` exit at once.
typedef double mf_f64x4 __attribute__((ext_vector_type(4)));
constexpr int kMfWaves = 4;

__global__ __launch_bounds__(kMfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void k_mfma_f64(double x, int waves, int iters, double *sink)
{
    const int64_t wave = (int64_t)blockIdx.x * kMfWaves + threadIdx.x / kWave;
    if (wave >= waves) return;
    mf_f64x4 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = (mf_f64x4){0.0, 0.0, 0.0, 0.0};
    // rounds in groups of four (iters is a multiple of 4): a rolled loop of
    // one round makes the compiler move the accumulators between register
    // files every round
    for (int i = 0; i < iters; i += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, x, acc[n], 0, 0, 0);
    }
    double s = 0.0;
#pragma unroll
    for (int n = 0; n < 8; ++n) s += (acc[n][0] + acc[n][1]) + (acc[n][2] + acc[n][3]);
    sink[wave * kWave + threadIdx.x % kWave] = s;
}

hipError_t launch_mfma_f64(double x, int waves, int iters, double *sink, hipStream_t s)
{
    hipLaunchKernelGGL(k_mfma_f64, dim3((waves + kMfWaves - 1) / kMfWaves), dim3(kMfWaves * kWave), 0, s, x, waves,
                       iters, sink);
    return hipGetLastError();
}

} // namespace swan
