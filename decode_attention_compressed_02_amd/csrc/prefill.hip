// prefill.hip -- convert a prefilled history into the hybrid cache (the step
// before decoding starts: the SWAN page's hybrid cache keeps the newest R tokens dense
// and every older one as its pruned sparse row).
//
// The key projection of a history is a dense contraction (tokens x 128
// rotated coordinates times the 128 x 128 P_QK of the head), carried out in
// double to match the decode-step projection, so it runs on the fp64 matrix
// cores (v_mfma_f64_16x16x4f64).  One workgroup of four waves per (chunk of
// 256 tokens, kv head, sequence):
//   0. P_QK of the head is staged in LDS as fp32 (64 KB, read once per
//      chunk) in a layout where a lane's eight 16-column blocks are
//      contiguous, and the 64 RoPE frequencies are computed once;
//   1. each wave takes 16-token tiles; lane l rotates the coordinate pairs
//      (c, c + 64) of token l % 16 for the 16 values of c that its MFMA k
//      column l / 16 covers, so the A operand never leaves registers;
//   2. 32 k steps x 8 column blocks of MFMA give the tile's 16 x 128
//      projected keys in double, each rounded once to fp16;
//   3. the wave places its tokens, eight at a time through a 2 KB LDS
//      stage: tokens older than len - R are pruned into their sparse rows
//      (the same wave-level top-k as the append kernel, the threshold
//      searches of four tokens' eight rows interleaved), the newest R go to
//      buffer slots t mod R.  Values are rounded from fp32 to fp16 directly.
// The result is identical to appending the tokens one at a time.  Keys are
// rotated and projected in double, as in the decode-step projection, so that
// their fp16 rounding (and with it the pruning) does not depend on float
// rounding of intermediate products.
//
// Operand layout of v_mfma_f64_16x16x4f64 (one wave): A[i][k] comes from lane
// i + 16 k, B[k][j] from lane j + 16 k, and result register r of lane l
// holds D[4 r + l / 16][l % 16].  The contraction index k of k step s maps
// to coordinate c(s, k) = 16 k + s for s < 16 and 64 + 16 k + (s - 16)
// otherwise, so both halves of a RoPE pair sit in the same lane.
#include "topk_rows.h"

namespace swan {

constexpr int kPfWaves = 4;            // waves per workgroup
constexpr int kPfTile = 16;            // tokens per MFMA tile (one wave)
constexpr int kPfChunk = 256;          // tokens per workgroup
constexpr int kPfBlocks = kD / 16;     // 16-column blocks of the output
constexpr int kPfHalf = kPfTile / 2;   // tokens per placement pass
constexpr int kPfGroup = 4;            // tokens whose rows are pruned together

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));

// coordinate of contraction index k (= lane / 16) in k step s
__device__ __forceinline__ int pf_coord(int s, int k) { return s < 16 ? 16 * k + s : kD / 2 + 16 * k + (s - 16); }

__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(PrefillArgs a)
{
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = min(a.len[b], a.max_len);
    const int c0 = chunk * kPfChunk;
    if (c0 >= T) return; // workgroup-uniform

    // P_QK[c][j] at pl[(c * 16 + j % 16) * 8 + j / 16]
    __shared__ __attribute__((aligned(16))) float pl[kD * 16 * kPfBlocks];
    __shared__ double theta[kD / 2];
    __shared__ uint16_t kst[kPfWaves][kPfHalf][kD];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    {
        const float *P = a.P + ((int64_t)(b / a.Bl) * a.H + h) * kD * kD;
        for (int e = tid * 4; e < kD * kD; e += kPfWaves * kWave * 4) {
            const pf_f32x4 p = *(const pf_f32x4 *)(P + e);
            const int c = e / kD, j = e % kD; // j % 4 == 0: the four columns share j / 16
#pragma unroll
            for (int x = 0; x < 4; ++x) pl[(c * 16 + (j + x) % 16) * kPfBlocks + (j + x) / 16] = p[x];
        }
        if (tid < kD / 2) theta[tid] = pow((double)a.base, -(double)tid / (double)(kD / 2));
    }
    __syncthreads();

    const int64_t u = (int64_t)b * a.H + h;
    const float *kr = a.k_raw + u * a.T_stride * kD;
    const float *vr = a.v_hat + u * a.T_stride * kD;
    const int kq = lane / 16, il = lane % 16; // MFMA k column and row of this lane's A element
    const int row_cap = a.geom.bs > 0 ? a.geom.max_blocks * a.geom.bs : a.geom.n_cap;
    const int c_end = min(T, c0 + kPfChunk);

    for (int t0 = c0 + wave * kPfTile; t0 < c_end; t0 += kPfWaves * kPfTile) {
        // ---- 1. rotated coordinates of token t0 + il: A[s] = x_rot[c(s, kq)]
        double A[32];
        {
            const int t = t0 + il;
            pf_f32x4 x0[4], x1[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                x0[v] = (pf_f32x4){0.f, 0.f, 0.f, 0.f};
                x1[v] = x0[v];
            }
            if (t < T) {
                const float *row = kr + (int64_t)t * kD + 16 * kq;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    x0[v] = *(const pf_f32x4 *)(row + 4 * v);
                    x1[v] = *(const pf_f32x4 *)(row + kD / 2 + 4 * v);
                }
            }
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                double sn, cs;
                sincos((double)t * theta[16 * kq + s], &sn, &cs);
                const double y0 = x0[s / 4][s % 4], y1 = x1[s / 4][s % 4];
                A[s] = y0 * cs - y1 * sn;
                A[16 + s] = y1 * cs + y0 * sn;
            }
        }

        // ---- 2. the tile times P_QK on the matrix cores
        f64x4 acc[kPfBlocks];
#pragma unroll
        for (int n = 0; n < kPfBlocks; ++n) acc[n] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const float *pc = pl + (pf_coord(s, kq) * 16 + il) * kPfBlocks;
            const pf_f32x4 p0 = *(const pf_f32x4 *)pc, p1 = *(const pf_f32x4 *)(pc + 4);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[s], (double)p0[n], acc[n], 0, 0, 0);
                acc[n + 4] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[s], (double)p1[n], acc[n + 4], 0, 0, 0);
            }
        }

        // ---- 3. place the tile's tokens, eight at a time
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            // register r = 2 hp + r2 of lane l holds token 4 r + l / 16 = 8 hp + (4 r2 + l / 16)
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int n = 0; n < kPfBlocks; ++n) kst[wave][4 * r2 + kq][16 * n + il] = d2h(acc[n][2 * hp + r2]);
            // the wave reads what its own lanes wrote (LDS runs a wave's accesses in order)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // four tokens (eight rows: key and value of each) at a time, so that
            // the eight top-k threshold searches interleave
            for (int g4 = 0; g4 < kPfHalf; g4 += kPfGroup) {
                const int tb = t0 + kPfHalf * hp + g4;
                if (tb >= T) break; // wave-uniform
                uint16_t lo[2 * kPfGroup], hi[2 * kPfGroup];
                int kk[2 * kPfGroup];
#pragma unroll
                for (int s = 0; s < kPfGroup; ++s) {
                    const int t = tb + s;
                    lo[2 * s] = kst[wave][g4 + s][lane];
                    hi[2 * s] = kst[wave][g4 + s][lane + 64];
                    const float *vt = vr + (int64_t)min(t, T - 1) * kD; // tokens past T are not placed
                    lo[2 * s + 1] = f2h(vt[lane]);
                    hi[2 * s + 1] = f2h(vt[lane + 64]);
                    kk[2 * s] = a.k;
                    kk[2 * s + 1] = a.k_v;
                }
                uint32_t thr[2 * kPfGroup];
                if (tb < T - a.R) wave_topk_threshold<2 * kPfGroup>(lo, hi, kk, thr); // some token is pruned
#pragma unroll
                for (int s = 0; s < kPfGroup; ++s) {
                    const int t = tb + s;
                    if (t >= T) break; // wave-uniform
#pragma unroll
                    for (int which = 0; which < 2; ++which) {
                        const int n = 2 * s + which;
                        if (t < T - a.R) {
                            const int64_t slot = t < row_cap ? row_slot_rt(a.geom, b, h, t) : -1;
                            const int ks = which ? a.geom.ks_v : a.geom.ks;
                            if (slot >= 0)
                                wave_write_topk(lane, lo[n], hi[n], thr[n], kk[n], ks,
                                                (which ? a.vidx : a.kidx) + slot * ks,
                                                (which ? a.vval : a.kval) + slot * ks * a.geom.vbytes, a.geom.vbytes);
                        } else {
                            uint16_t *buf = (which ? a.vbuf : a.kbuf) + (u * a.R + t % a.R) * kD;
                            buf[lane] = lo[n];
                            buf[lane + 64] = hi[n];
                        }
                    }
                }
            }
            // the stage is rewritten by the next pass only after these reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s)
{
    const dim3 grid((a.max_len + kPfChunk - 1) / kPfChunk, a.H, a.B);
    hipLaunchKernelGGL(k_prefill, grid, dim3(kPfWaves * kWave), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
