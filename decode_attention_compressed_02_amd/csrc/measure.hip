// measure.hip -- the streaming-read yardstick of swan_measure.h: how fast
// this GPU reads a buffer once from HBM, the ceiling for a decode step that
// must read its whole cache every step.
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

} // namespace swan
