// decode.hip -- hybrid decode attention (SWAN section 4.2 and appendix A.2,
// steps 2-4): scores of the rotated query against the sparse history (an
// indexed gather of q_hat) and the dense buffer, one softmax over both, and
// the output accumulated from sparse values (scatter-add at the stored
// indices) and dense values.
//
// Pass 1 (k_split): one wavefront per (split, kv head, sequence).  The wave
// serves all g query heads of the GQA group, so every sparse row streamed
// from HBM is used g times.  Splits 0..S_sparse-1 cover consecutive ranges
// of sparse rows; the remaining splits cover the dense buffer.  Each wave
// keeps an online softmax (running max m, running sum l) and writes
// (m, l, unnormalised output) per query head.
//
// Sparse streaming layout: a row is k_stride entries, 8 entries per lane,
// LPT = k_stride / 8 lanes per token, 64 / LPT tokens per wave iteration.
// Lane i of the wave loads bytes [8i, 8i+8) of the iteration's index block
// and bytes [16i, 16i+16) of its value block, so each wave load instruction
// reads one contiguous 512 B / 1 KiB span of a plane.
//
// The scaled q_hat of the group sits in LDS as qs[c][g] (one 16-byte read per
// gathered index for g = 4).  The output accumulator sits in LDS as
// acc[c][g] and is updated with LDS float atomics, since lanes of different
// tokens may hit the same coordinate in one instruction.  Scores are in
// base-2 units (q_hat pre-scaled by log2(e)/sqrt(d_h)).  The running max is
// raised only when a score exceeds it by more than kRescaleSlack, so the
// accumulator rescale (a pass over LDS) is rare; weights stay below
// 2^kRescaleSlack.
//
// Pass 2 (k_reduce): one workgroup per (query head, sequence) merges the S
// partials with the usual log-sum-exp weights.
#include "swan_internal.h"

namespace swan {

constexpr float kRescaleSlack = 8.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int G>
__device__ __forceinline__ void lds_q(const float *__restrict__ qs, int c, float (&q)[G])
{
    if constexpr (G == 1) {
        q[0] = qs[c];
    } else if constexpr (G == 2) {
        const f32x2 t = *(const f32x2 *)(qs + 2 * c);
        q[0] = t.x;
        q[1] = t.y;
    } else if constexpr (G == 4) {
        const f32x4 t = *(const f32x4 *)(qs + 4 * c);
        q[0] = t.x;
        q[1] = t.y;
        q[2] = t.z;
        q[3] = t.w;
    } else {
        const f32x4 t0 = *(const f32x4 *)(qs + 8 * c), t1 = *(const f32x4 *)(qs + 8 * c + 4);
        q[0] = t0.x; q[1] = t0.y; q[2] = t0.z; q[3] = t0.w;
        q[4] = t1.x; q[5] = t1.y; q[6] = t1.z; q[7] = t1.w;
    }
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ void lds_add(float *p, float v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct Chunk {
    uint64_t ki, vi;
    u32x4 kv, vv;
};

template <int G, int LPT, bool PAGED>
__global__ __launch_bounds__(64) void k_split(SplitArgs a)
{
    constexpr int TPC = kWave / LPT; // tokens per wave iteration
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    __shared__ __attribute__((aligned(16))) float qs[kD * G];
    __shared__ __attribute__((aligned(16))) float acc[kD * G];

    const int ctx = a.pos[b] + 1; // tokens attended; <= 0 for an inactive sequence
    const int n = min(ctx > a.R ? ctx - a.R : 0, a.row_cap);
    const int fill = max(0, min(ctx, a.R));

    const float *qsrc = a.q_hat + ((int64_t)b * a.N_h + h * G) * kD;
    for (int i = lane; i < kD * G; i += kWave) {
        const int hh = i / kD, c = i % kD;
        qs[c * G + hh] = qsrc[i] * kScoreScaleLog2;
        acc[i] = 0.f;
    }
    __syncthreads();

    float m[G], l[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
    }
    // partial (b, h*G + hh, split) lives at index pbase + hh * S
    const int64_t pbase = ((int64_t)b * a.N_h + h * G) * a.S + split;

    if (split < a.S_sparse) {
        const int t0 = split * a.TPS, t1 = min(t0 + a.TPS, n);
        const int tl = lane / LPT, sub = lane % LPT;
        auto load = [&](int r0, Chunk &c) {
            const int r = r0 + tl;
            const int64_t off = r < t1 ? row_offset<PAGED>(a.geom, b, h, r) : -1;
            if (off >= 0) {
                const int64_t e = off + sub * 8;
                c.ki = *(const uint64_t *)(a.kidx + e);
                c.kv = *(const u32x4 *)(a.kval + e);
                c.vi = *(const uint64_t *)(a.vidx + e);
                c.vv = *(const u32x4 *)(a.vval + e);
            } else {
                c.ki = c.vi = 0;
                c.kv = c.vv = (u32x4){0u, 0u, 0u, 0u};
            }
        };
        Chunk nx;
        if (t0 < t1) load(t0, nx);
        for (int r0 = t0; r0 < t1; r0 += TPC) {
            const Chunk cur = nx;
            if (r0 + TPC < t1) load(r0 + TPC, nx);
            const bool valid = r0 + tl < t1;

            // scores: gather q_hat at the stored key indices
            float s[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
            const half8 kvh = __builtin_bit_cast(half8, cur.kv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = (int)((cur.ki >> (8 * i)) & 0xffu);
                float q[G];
                lds_q<G>(qs, c, q);
                const float v = (float)kvh[i];
#pragma unroll
                for (int hh = 0; hh < G; ++hh) s[hh] = fmaf(q[hh], v, s[hh]);
            }
#pragma unroll
            for (int o = 1; o < LPT; o <<= 1)
#pragma unroll
                for (int hh = 0; hh < G; ++hh) s[hh] += __shfl_xor(s[hh], o);
            bool need = false;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                if (!valid) s[hh] = -INFINITY;
                need |= s[hh] > m[hh] + kRescaleSlack;
            }
            if (__any(need)) { // wave-uniform
                float f[G];
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float mn = fmaxf(m[hh], wave_max(s[hh]));
                    f[hh] = exp2f(m[hh] - mn);
                    m[hh] = mn;
                    l[hh] *= f[hh];
                }
                float fl = f[0];
#pragma unroll
                for (int hh = 1; hh < G; ++hh)
                    if (lane % G == hh) fl = f[hh];
                __syncthreads();
                for (int i = lane; i < kD * G; i += kWave) acc[i] *= fl; // i % G == lane % G
                __syncthreads();
            }
            float w[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                w[hh] = exp2f(s[hh] - m[hh]);
                if (sub == 0) l[hh] += w[hh];
            }
            // outputs: scatter-add weighted values at the stored value indices
            if (valid) {
                const half8 vvh = __builtin_bit_cast(half8, cur.vv);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c = (int)((cur.vi >> (8 * i)) & 0xffu);
                    const float v = (float)vvh[i];
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) lds_add(acc + c * G + hh, w[hh] * v);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float lt = wave_sum(l[hh]);
            if (lane == 0) {
                a.part_ml[(pbase + hh * a.S) * 2] = m[hh];
                a.part_ml[(pbase + hh * a.S) * 2 + 1] = lt;
            }
            for (int c = lane; c < kD; c += kWave) a.part_o[(pbase + hh * a.S) * kD + c] = acc[c * G + hh];
        }
    } else {
        // dense buffer: 16 lanes per token, 8 coordinates per lane, 4 tokens per iteration
        const int t0 = (split - a.S_sparse) * kDenseSplit, t1 = min(t0 + kDenseSplit, fill);
        const int tl = lane / 16, c0 = (lane % 16) * 8;
        float qr[8][G], ar[8][G];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                qr[i][hh] = qs[(c0 + i) * G + hh];
                ar[i][hh] = 0.f;
            }
        const int64_t ub = ((int64_t)b * a.H + h) * a.R * kD + c0;
        for (int t = t0; t < t1; t += 4) {
            const int tok = t + tl;
            const bool valid = tok < t1;
            u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (valid) {
                kk = *(const u32x4 *)(a.kbuf + ub + (int64_t)tok * kD);
                vv = *(const u32x4 *)(a.vbuf + ub + (int64_t)tok * kD);
            }
            const half8 kh = __builtin_bit_cast(half8, kk), vh = __builtin_bit_cast(half8, vv);
            float s[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                s[hh] = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) s[hh] = fmaf(qr[i][hh], (float)kh[i], s[hh]);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1)
#pragma unroll
                for (int hh = 0; hh < G; ++hh) s[hh] += __shfl_xor(s[hh], o);
            bool need = false;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                if (!valid) s[hh] = -INFINITY;
                need |= s[hh] > m[hh] + kRescaleSlack;
            }
            if (__any(need)) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float mn = fmaxf(m[hh], wave_max(s[hh]));
                    const float f = exp2f(m[hh] - mn);
                    m[hh] = mn;
                    l[hh] *= f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ar[i][hh] *= f;
                }
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float w = exp2f(s[hh] - m[hh]);
                if ((lane % 16) == 0) l[hh] += w;
#pragma unroll
                for (int i = 0; i < 8; ++i) ar[i][hh] = fmaf(w, (float)vh[i], ar[i][hh]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                ar[i][hh] += __shfl_xor(ar[i][hh], 16);
                ar[i][hh] += __shfl_xor(ar[i][hh], 32);
            }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float lt = wave_sum(l[hh]);
            if (lane == 0) {
                a.part_ml[(pbase + hh * a.S) * 2] = m[hh];
                a.part_ml[(pbase + hh * a.S) * 2 + 1] = lt;
            }
            if (tl == 0) {
                float *dst = a.part_o + (pbase + hh * a.S) * kD + c0;
                *(f32x4 *)dst = (f32x4){ar[0][hh], ar[1][hh], ar[2][hh], ar[3][hh]};
                *(f32x4 *)(dst + 4) = (f32x4){ar[4][hh], ar[5][hh], ar[6][hh], ar[7][hh]};
            }
        }
    }
}

// Merge the S partials of one (query head, sequence).  Thread c owns output
// coordinate c.  An all-empty head (inactive sequence) yields zeros.
__global__ __launch_bounds__(128) void k_reduce(ReduceArgs a)
{
    const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const int64_t base = ((int64_t)b * a.N_h + hq) * a.S;
    float mx = -INFINITY;
    for (int s = 0; s < a.S; ++s) mx = fmaxf(mx, a.part_ml[(base + s) * 2]);
    float o = 0.f, L = 0.f;
    if (mx != -INFINITY) {
        for (int s = 0; s < a.S; ++s) {
            const float ms = a.part_ml[(base + s) * 2];
            if (ms == -INFINITY) continue;
            const float w = exp2f(ms - mx);
            L = fmaf(w, a.part_ml[(base + s) * 2 + 1], L);
            o = fmaf(w, a.part_o[(base + s) * kD + c], o);
        }
        o /= L;
    }
    a.o_hat[((int64_t)b * a.N_h + hq) * kD + c] = o;
}

template <int G, bool PAGED>
static hipError_t launch_split_g(const SplitArgs &a, hipStream_t s)
{
    const dim3 grid(a.S, a.H, a.B), block(kWave);
    switch (a.geom.ks / 8) {
    case 1: hipLaunchKernelGGL((k_split<G, 1, PAGED>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_split<G, 2, PAGED>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_split<G, 4, PAGED>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_split<G, 8, PAGED>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_split<G, 16, PAGED>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_split(const SplitArgs &a, int g, hipStream_t s)
{
    const bool paged = a.geom.bs > 0;
    switch (g) {
    case 1: return paged ? launch_split_g<1, true>(a, s) : launch_split_g<1, false>(a, s);
    case 2: return paged ? launch_split_g<2, true>(a, s) : launch_split_g<2, false>(a, s);
    case 4: return paged ? launch_split_g<4, true>(a, s) : launch_split_g<4, false>(a, s);
    case 8: return paged ? launch_split_g<8, true>(a, s) : launch_split_g<8, false>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_reduce, dim3(a.N_h, a.B), dim3(kD), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
