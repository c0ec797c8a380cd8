// prefill.hip -- convert a prefilled history into the hybrid cache (the step
// before decoding starts: the SWAN page's hybrid cache keeps the newest R
// tokens dense and every older one as its pruned sparse row).
//
// The key projection of a history is a dense contraction (tokens x 128
// rotated coordinates times the 128 x 128 P_QK of the head), carried out in
// double to match the decode-step projection, so it runs on the fp64 matrix
// cores (v_mfma_f64_16x16x4f64).  One workgroup of eight waves per chunk of
// 128 to 512 tokens of one (kv head, sequence) (shorter chunks for small
// batches; only chunks that hold tokens are numbered, so ragged batches leave
// no idle workgroups among the busy ones):
//   0. P_QK of the head is staged in LDS as fp32 (64 KB, read once per
//      chunk) in a layout where a lane's eight 16-column blocks are
//      contiguous, and the 64 RoPE frequencies are computed once;
//   1. each wave takes 16-token tiles; lane l rotates the coordinate pairs
//      (c, c + 64) of token l % 16 for the 16 values of c that its MFMA k
//      column l / 16 covers, so the A operand never leaves registers;
//   2. 32 k steps x 8 column blocks of MFMA give the tile's 16 x 128
//      projected keys in double;
//   3. eight tokens at a time, their keys (rounded once to fp16, branch-free:
//      fp16_round.h) and values (fp32 -> fp16, loaded one pass ahead) are
//      staged in LDS as 16 rows; tokens older than len - R are pruned into
//      their sparse rows, the newest R go to buffer slots t mod R.
//
// Pruning (SWAN page, pruning paragraph: a vector keeps its k coordinates of
// largest magnitude) takes four lanes a row, lane 4 r + q holding
// coordinates 32 q .. 32 q + 31 of row r as packed fp16, all in VALU
// arithmetic: the k-th largest magnitude T is found bit by bit (the largest T
// with at least k magnitudes >= T; a packed 16-bit subtract's sign bits mark
// the magnitudes below a candidate and v_sad_u16 adds them up), then every
// coordinate above T is kept together with the first k - #(above T) equal to
// T in index order, the ranking of the append kernel's wave_prune_row.  Each
// lane writes its kept entries, in index order, to the row's place in an LDS
// output stage (the others to a scratch byte, so no lane branches), and
// whole rows go to their slots with 32-bit stores.
//
// The result is identical to appending the tokens one at a time.  Keys are
// rotated and projected in double, as in the decode-step projection, so that
// their fp16 rounding (and with it the pruning) does not depend on float
// rounding of intermediate products; the rotation's sine and cosine come from
// rope_trig.h (within ~1e-16 of the true values, as a library sincos).
//
// Operand layout of v_mfma_f64_16x16x4f64 (one wave): A[i][k] comes from lane
// i + 16 k, B[k][j] from lane j + 16 k, and result register r of lane l
// holds D[4 r + l / 16][l % 16].  The contraction index k of k step s maps
// to coordinate c(s, k) = 16 k + s for s < 16 and 64 + 16 k + (s - 16)
// otherwise, so both halves of a RoPE pair sit in the same lane.
#include <type_traits>

#include "fp16_round.h"
#include "rope_trig.h"
#include "swan_internal.h"

namespace swan {

constexpr int kPfWaves = 8;            // waves per workgroup
constexpr int kPfTile = 16;            // tokens per MFMA tile (one wave)
constexpr int kPfChunkMax = 512;       // tokens per workgroup (fewer when the grid would be small)
constexpr int kPfComputeUnits = 256;   // of an MI355X
constexpr int kPfBlocks = kD / 16;     // 16-column blocks of the output
constexpr int kPfHalf = kPfTile / 2;   // tokens per placement pass
constexpr int kPfRow = kD + 8;         // staged row stride in fp16 (272 bytes: the quarter reads meet no bank twice)
constexpr int kPfOut = 3 * kD + 16;    // bytes of a pruned row in the output stage: indices, values, a scratch slot
constexpr int kPfTrash = 3 * kD;       // the scratch slot: entries that are not kept are written there

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pf_u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t pf_u16x2 __attribute__((ext_vector_type(2)));
typedef float pf_f32x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ uint32_t pf_dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// coordinate of contraction index k (= lane / 16) in k step s
__device__ __forceinline__ int pf_coord(int s, int k) { return s < 16 ? 16 * k + s : kD / 2 + 16 * k + (s - 16); }

__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(PrefillArgs a,
                                                                                                   int chunk_len)
{
    // Work item = one chunk of one (sequence, kv head) that holds tokens,
    // numbered sequence by sequence, head by head, chunk by chunk: the chunks
    // of ragged sequences stay contiguous in the grid (so consecutive
    // workgroups, spread over the XCDs in turn, all have work) and the grid's
    // surplus workgroups, all at its end, exit at once.  Wave 0 finds the
    // item's sequence from a prefix sum of the sequences' chunk counts.
    __shared__ int64_t item_base;
    __shared__ int item_b, item_chunks;
    {
        const int64_t item = blockIdx.x;
        if (threadIdx.x < kWave) {
            const int ln = threadIdx.x;
            int64_t run = 0;
            int found = -1, fn = 0;
            int64_t fbase = 0;
            for (int base = 0; base < a.B && found < 0; base += kWave) {
                const int bb = base + ln;
                const int n = bb < a.B ? (max(0, min(a.len[bb], a.max_len)) + chunk_len - 1) / chunk_len : 0;
                const int64_t cnt = (int64_t)n * a.H;
                int64_t incl = cnt; // inclusive prefix over the lanes
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const int64_t t = __shfl_up(incl, d);
                    if (ln >= d) incl += t;
                }
                incl += run;
                const uint64_t hit = __ballot(bb < a.B && incl > item);
                if (hit) {
                    const int l = __builtin_ctzll(hit);
                    found = base + l;
                    fbase = __shfl(incl - cnt, l);
                    fn = __shfl(n, l);
                }
                run = __shfl(incl, kWave - 1);
            }
            if (ln == 0) {
                item_b = found;
                item_base = fbase;
                item_chunks = fn;
            }
        }
        __syncthreads();
    }
    if (item_b < 0) return; // workgroup-uniform: past the last item
    const int b = item_b;
    const int h = (int)(((int64_t)blockIdx.x - item_base) / item_chunks);
    const int chunk = (int)(((int64_t)blockIdx.x - item_base) % item_chunks);
    const int T = min(a.len[b], a.max_len);
    const int c0 = chunk * chunk_len;

    // P_QK[c][j] at pl[(c * 16 + j % 16) * 8 + j / 16]
    __shared__ __attribute__((aligned(16))) float pl[kD * 16 * kPfBlocks];
    __shared__ double theta[kD / 2];
    __shared__ __attribute__((aligned(16))) uint16_t kst[kPfWaves][2 * kPfHalf][kPfRow];
    // pruned rows as stored: indices at [0, 128), values (vbytes each) from 128
    __shared__ __attribute__((aligned(16))) uint8_t pout[kPfWaves][2 * kPfHalf][kPfOut];
    __shared__ int64_t pslot[kPfWaves][kPfHalf]; // row slot of each token of a pass (-1: not pruned)

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
    const int c_end = min(T, c0 + chunk_len);

    for (int t0 = c0 + wave * kPfTile; t0 < c_end; t0 += kPfWaves * kPfTile) {
        // values of the tile's first eight tokens (tokens past T are not placed)
        pf_f32x2 vpre[kPfHalf];
#pragma unroll
        for (int s = 0; s < kPfHalf; ++s) vpre[s] = *(const pf_f32x2 *)(vr + (int64_t)min(t0 + s, T - 1) * kD + 2 * lane);
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
                rope_sincos((double)t * theta[16 * kq + s], sn, cs);
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
                for (int n = 0; n < kPfBlocks; ++n) kst[wave][4 * r2 + kq][16 * n + il] = d2h_odd(acc[n][2 * hp + r2]);
            // values of the same eight tokens, rounded to fp16, in rows 8..15 (two
            // coordinates a lane, one 32-bit LDS write); the next pass's values
            // are loaded now, to arrive while this pass is pruned
#pragma unroll
            for (int s = 0; s < kPfHalf; ++s) {
                const uint32_t lo16 = f2h(vpre[s].x), hi16 = f2h(vpre[s].y);
                *(uint32_t *)&kst[wave][kPfHalf + s][2 * lane] = lo16 | (hi16 << 16);
            }
            if (hp == 0) {
#pragma unroll
                for (int s = 0; s < kPfHalf; ++s)
                    vpre[s] = *(const pf_f32x2 *)(vr + (int64_t)min(t0 + kPfHalf + s, T - 1) * kD + 2 * lane);
            }
            // the wave reads what its own lanes wrote (LDS runs a wave's accesses in order)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int tb = t0 + kPfHalf * hp;
            if (tb >= T) continue; // wave-uniform
            // ---- prune the 16 staged rows, four lanes a row: lane 4 r + q holds
            // coordinates 32 q .. 32 q + 31 of row r (rows 0..7 the keys, 8..15 the
            // values of tokens tb .. tb + 7) as packed fp16
            if (tb < T - a.R) { // some token of the pass is pruned (wave-uniform)
                const int r = lane >> 2, q = lane & 3;
                const int kr = r < kPfHalf ? a.k : a.k_v, ksr = r < kPfHalf ? a.geom.ks : a.geom.ks_v;
                uint32_t x[16], m[16];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const pf_u32x4 w4 = *(const pf_u32x4 *)&kst[wave][r][32 * q + 8 * v];
                    x[4 * v] = w4.x;
                    x[4 * v + 1] = w4.y;
                    x[4 * v + 2] = w4.z;
                    x[4 * v + 3] = w4.w;
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) m[j] = x[j] & 0x7fff7fffu;
                // Counting by sums: for 15-bit magnitudes m and a candidate c, the packed
                // 16-bit difference m - c wraps by 2^16 exactly when m < c, so the sum of
                // the 32 differences (v_sad_u16 adds both halves, no wrap in 32 bits) is
                // sum(m) - 32 c + 2^16 #(m < c): one subtract and one add a word.
                uint32_t sm4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int j = 0; j < 16; ++j) sm4[j & 3] = __builtin_amdgcn_sad_u16(m[j], 0u, sm4[j & 3]);
                const uint32_t sum_m = (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
                auto count_below = [&](uint32_t c) -> int { // #(m < c) over the lane's 32 coordinates
                    const pf_u16x2 cp = {(uint16_t)c, (uint16_t)c};
                    uint32_t acc4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        acc4[j & 3] = __builtin_amdgcn_sad_u16(
                            __builtin_bit_cast(uint32_t, __builtin_bit_cast(pf_u16x2, m[j]) - cp), 0u, acc4[j & 3]);
                    return (int)(((acc4[0] + acc4[1]) + (acc4[2] + acc4[3]) + 32u * c - sum_m) >> 16);
                };
                // the k-th largest magnitude T: the largest T with at least k
                // magnitudes >= T, bit by bit
                uint32_t Tt = 0;
#pragma unroll
                for (int bit = 14; bit >= 0; --bit) {
                    const uint32_t c = Tt | (1u << bit);
                    uint32_t lt = (uint32_t)count_below(c);
                    lt += pf_dpp<0xB1>(lt);
                    lt += pf_dpp<0x4E>(lt);
                    if (kD - (int)lt >= kr) Tt = c;
                }
                // kept: every magnitude above T, then the first need = k - #(above T)
                // equal to T in index order (lower quarters first)
                const int n_lt = count_below(Tt), n_gt = 32 - count_below(Tt + 1), n_eq = 32 - n_gt - n_lt;
                // quad sums and exclusive prefixes (lane q of the row's quad)
                const int g1 = (int)pf_dpp<0x00>(n_gt), g2 = (int)pf_dpp<0x55>(n_gt), g3 = (int)pf_dpp<0xAA>(n_gt),
                          g4 = (int)pf_dpp<0xFF>(n_gt);
                const int e1 = (int)pf_dpp<0x00>(n_eq), e2 = (int)pf_dpp<0x55>(n_eq), e3 = (int)pf_dpp<0xAA>(n_eq),
                          e4 = (int)pf_dpp<0xFF>(n_eq);
                const int need = kr - (g1 + g2 + g3 + g4);
                const int eq_before = (q > 0 ? e1 : 0) + (q > 1 ? e2 : 0) + (q > 2 ? e3 : 0);
                const int allow = min(max(need - eq_before, 0), n_eq);
                const int mine = n_gt + allow;
                const int k1 = (int)pf_dpp<0x00>(mine), k2 = (int)pf_dpp<0x55>(mine), k3 = (int)pf_dpp<0xAA>(mine);
                int pos = (q > 0 ? k1 : 0) + (q > 1 ? k2 : 0) + (q > 2 ? k3 : 0);
                uint8_t *orow = pout[wave][r];
                const int vb = a.geom.vbytes;
                // every lane writes: kept entries at their place, the rest to the scratch
                // slot; VB (the value width) is a compile-time constant in each loop
                auto put = [&](auto VB, int i, uint32_t v, bool keep) {
                    constexpr int kVB = decltype(VB)::value;
                    const int io = keep ? pos : kPfTrash, vo = keep ? kD + kVB * pos : kPfTrash + 2;
                    orow[io] = (uint8_t)(32 * q + i);
                    if constexpr (kVB == 1)
                        orow[vo] = h2e4m3((uint16_t)v);
                    else
                        *(uint16_t *)(orow + vo) = (uint16_t)v;
                    pos += keep ? 1 : 0;
                };
                auto assemble = [&](auto VB) {
                    if (__all(need == e1 + e2 + e3 + e4)) {
                        // no row splits its coordinates equal to T (the usual case): each
                        // keeps exactly the magnitudes >= T
#pragma unroll
                        for (int i = 0; i < 32; ++i) {
                            const uint32_t v = (i & 1) ? (x[i / 2] >> 16) : (x[i / 2] & 0xffffu);
                            put(VB, i, v, (v & 0x7fffu) >= Tt);
                        }
                    } else {
                        int eq_seen = 0;
#pragma unroll
                        for (int i = 0; i < 32; ++i) {
                            const uint32_t v = (i & 1) ? (x[i / 2] >> 16) : (x[i / 2] & 0xffffu);
                            const uint32_t mag = v & 0x7fffu;
                            const bool is_eq = mag == Tt;
                            put(VB, i, v, mag > Tt || (is_eq && eq_seen < allow));
                            eq_seen += is_eq ? 1 : 0;
                        }
                    }
                };
                if (vb == 1)
                    assemble(std::integral_constant<int, 1>());
                else
                    assemble(std::integral_constant<int, 2>());
                // padding entries k .. ks - 1: index 0, value +0
                for (int e = kr + q; e < ksr; e += 4) {
                    orow[e] = 0;
                    if (vb == 1)
                        orow[kD + e] = 0;
                    else
                        *(uint16_t *)(orow + kD + 2 * e) = 0;
                }
                if (lane < kPfHalf) {
                    const int t = tb + lane;
                    pslot[wave][lane] = (t < T - a.R && t < row_cap) ? row_slot_rt(a.geom, b, h, t) : -1;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // whole rows to their slots, one dword a lane (row widths are powers of two)
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    const int ksw = which ? a.geom.ks_v : a.geom.ks;
                    const int wsh = __builtin_ctz((unsigned)ksw) - 2;       // log2 of the index row's dwords
                    const int vsh = wsh + (vb == 2 ? 1 : 0);                // log2 of the value row's dwords
                    uint8_t *iplane = which ? a.vidx : a.kidx, *vplane = which ? a.vval : a.kval;
                    for (int e = lane; e < (kPfHalf << wsh); e += kWave) {
                        const int sidx = e >> wsh, w = e & ((1 << wsh) - 1);
                        const int64_t slot = pslot[wave][sidx];
                        if (slot >= 0)
                            *(uint32_t *)(iplane + slot * ksw + 4 * w) =
                                *(const uint32_t *)(pout[wave][which * kPfHalf + sidx] + 4 * w);
                    }
                    for (int e = lane; e < (kPfHalf << vsh); e += kWave) {
                        const int sidx = e >> vsh, w = e & ((1 << vsh) - 1);
                        const int64_t slot = pslot[wave][sidx];
                        if (slot >= 0)
                            *(uint32_t *)(vplane + slot * ksw * vb + 4 * w) =
                                *(const uint32_t *)(pout[wave][which * kPfHalf + sidx] + kD + 4 * w);
                    }
                }
            }
            // ---- the newest R tokens go to the buffer
            if (tb + kPfHalf > T - a.R) {
                for (int s = 0; s < kPfHalf; ++s) {
                    const int t = tb + s;
                    if (t >= T) break; // wave-uniform
                    if (t < T - a.R) continue;
#pragma unroll
                    for (int which = 0; which < 2; ++which) {
                        const int row = which * kPfHalf + s;
                        uint16_t *buf = (which ? a.vbuf : a.kbuf) + (u * a.R + t % a.R) * kD;
                        buf[lane] = kst[wave][row][lane];
                        buf[lane + 64] = kst[wave][row][lane + 64];
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
    // the longest chunk (P_QK staged once per chunk) that still gives about
    // two workgroups per compute unit; one 16-token tile per wave at least
    int chunk = kPfChunkMax;
    while (chunk > kPfWaves * kPfTile &&
           (int64_t)((a.max_len + chunk - 1) / chunk) * a.H * a.B < 2 * kPfComputeUnits)
        chunk /= 2;
    // one workgroup per chunk of the longest sequence for every (sequence,
    // head): at least as many as there are work items
    const int64_t items = (int64_t)((a.max_len + chunk - 1) / chunk) * a.H * a.B;
    if (items > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)items);
    hipLaunchKernelGGL(k_prefill, grid, dim3(kPfWaves * kWave), 0, s, a, chunk);
    return hipGetLastError();
}

} // namespace swan
