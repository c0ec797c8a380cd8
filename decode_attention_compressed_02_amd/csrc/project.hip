// project.hip -- runtime projection of the new query and key (SWAN page,
// projection-absorption paragraphs: RoPE is position dependent, so RoPE(x)
// P_QK cannot be folded into the weights and runs every decode step).
//
// One workgroup of 512 threads per (kv head, sequence).  The g query vectors
// of the GQA group and the new key are rotated by RoPE into LDS; thread
// (quarter, j) then applies rows 32 quarter .. 32 quarter + 31 of P_QK to all
// g + 1 vectors for output coordinate j (loads of a row are 512 contiguous
// bytes across the 128 threads of a quarter; P_QK is L2-resident across the
// sequences of a batch), and the four partial sums meet in LDS.  The 4 d_h^2
// FLOPs per head of SWAN appendix A.2 are tiny next to the decode stream: the
// kernel is latency-bound, so the row walk is cut four ways and every load is
// issued before the first barrier.
//
// The arithmetic is in double: the new key is rounded once to fp16 and its
// top-k coordinates are chosen on those fp16 magnitudes, so a key computed
// in float could round one ulp away from the exact product and change which
// coordinates survive pruning.  In double the result is the correctly
// rounded fp16 of the exact value except within ~1e-16 of a midpoint.
#include "fp16_round.h"
#include "rope_trig.h"
#include "swan_internal.h"

namespace swan {

constexpr int kProjThreads = 512;
constexpr int kProjRows = kD / (kProjThreads / kD); // rows of P per thread group

// With APPEND the workgroup also appends the unit's new key and value.  The
// value needs no projection and the token leaving the buffer needs nothing
// of the new one, so the last two waves append the value and evict the
// oldest key while the rotation angles are computed; only the new key's
// placement waits for the projection.  Every load that depends on no other
// (raw vectors, rows of P_QK, the old buffer entries) is issued at the start.
// Block that sequence b's append writes this step, from the launch's table
// entries (slots are distinct, so at most one matches), or kTableBlock when
// the entries do not set that slot (the table then holds it and this launch
// does not write it).  Run by a whole wave; every lane gets the answer.
__device__ int wave_append_block(const StepUpdateArgs &u, const AppendArgs &ap, int b, int lane)
{
    const int p = ap.pos[b];
    const int r = ap.R > 0 ? p - ap.R : p; // sparse row written this step
    if (p < 0 || r < 0 || r / ap.geom.bs >= ap.geom.max_blocks) return kTableBlock;
    const int slot = b * ap.geom.max_blocks + r / ap.geom.bs;
    int hit = -1;
    for (int t = lane; t < u.n_entries; t += kWave)
        if (u.entry[t][0] == slot) hit = t;
    const uint64_t m = __ballot(hit >= 0);
    if (!m) return kTableBlock;
    return u.entry[__builtin_amdgcn_readlane(hit, __builtin_ctzll(m))][1];
}

// (u: the launch's table update on a paged step, whose entries give the
// appended rows' blocks; nullptr to read the block table)
template <int G, bool APPEND>
__device__ __forceinline__ void project_unit(const ProjectArgs &a, const AppendArgs &ap, int h, int b,
                                             const StepUpdateArgs *u)
{
    const int tid = threadIdx.x;
    const int j = tid % kD, quarter = tid / kD, wave = tid / kWave, lane = tid % kWave;
    constexpr int kWaves = kProjThreads / kWave;
    __shared__ double xs[G + 1][kD];
    __shared__ double part[kProjThreads / kD - 1][G + 1][kD];
    __shared__ double cs[kD / 2], sn[kD / 2];
    __shared__ uint16_t khs[APPEND ? kD : 1];

    // RoPE items (vector v, pair i) = tid, tid + 512, ...: v < G are the
    // query heads of the group, v = G the key
    constexpr int kItems = (G + 1) * (kD / 2), kPer = (kItems + kProjThreads - 1) / kProjThreads;
    float x0[kPer], x1[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int e = tid + r * kProjThreads, v = e / (kD / 2), i = e % (kD / 2);
        x0[r] = x1[r] = 0.f;
        if (e < kItems) {
            const float *x = (v < G) ? a.q + ((int64_t)b * a.N_h + h * G + v) * kD : a.k + ((int64_t)b * a.H + h) * kD;
            x0[r] = x[i];
            x1[r] = x[i + kD / 2];
        }
    }
    const int c0 = quarter * kProjRows;
    float pr[kProjRows];
    {
        const float *P = a.P + ((int64_t)(b / a.Bl) * a.H + h) * kD * kD + (int64_t)c0 * kD + j;
#pragma unroll
        for (int u = 0; u < kProjRows; ++u) pr[u] = P[u * kD];
    }
    if constexpr (APPEND) {
        if (wave == kWaves - 1) {
            const int64_t un = (int64_t)b * ap.H + h;
            const int blk = u ? wave_append_block(*u, ap, b, lane) : kTableBlock;
            append_token(ap, b, h, 1, lane, f2h(ap.v_hat[un * kD + lane]), f2h(ap.v_hat[un * kD + lane + 64]), blk);
        } else if (wave == kWaves - 2) {
            evict_token(ap, b, h, 0, lane, u ? wave_append_block(*u, ap, b, lane) : kTableBlock);
        }
    }
    if (tid < kD / 2) {
        // angle in double: at positions ~1e5 a float angle is off by ~1e-2 rad
        const double theta = pow((double)a.base, -(double)tid / (double)(kD / 2));
        const int p = max(a.pos[b], 0);
        double sv, cv;
        rope_sincos((double)p * theta, sv, cv);
        cs[tid] = cv;
        sn[tid] = sv;
    }
    __syncthreads();
    // RoPE: pair (i, i + 64) rotated by angle_i
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int e = tid + r * kProjThreads, v = e / (kD / 2), i = e % (kD / 2);
        if (e < kItems) {
            const double y0 = x0[r], y1 = x1[r];
            xs[v][i] = y0 * cs[i] - y1 * sn[i];
            xs[v][i + kD / 2] = y1 * cs[i] + y0 * sn[i];
        }
    }
    __syncthreads();

    // thread (quarter, j): rows c0 .. c0 + 31 of P_QK for output coordinate j
    double acc[G + 1];
#pragma unroll
    for (int v = 0; v < G + 1; ++v) acc[v] = 0.0;
#pragma unroll
    for (int u = 0; u < kProjRows; ++u)
#pragma unroll
        for (int v = 0; v < G + 1; ++v) acc[v] = fma(xs[v][c0 + u], (double)pr[u], acc[v]);
    if (quarter > 0) {
#pragma unroll
        for (int v = 0; v < G + 1; ++v) part[quarter - 1][v][j] = acc[v];
    }
    __syncthreads();
    if (quarter == 0) {
#pragma unroll
        for (int v = 0; v < G + 1; ++v)
#pragma unroll
            for (int r = 0; r < kProjThreads / kD - 1; ++r) acc[v] += part[r][v][j];
#pragma unroll
        for (int v = 0; v < G; ++v) a.q_hat[((int64_t)b * a.N_h + h * G + v) * kD + j] = (float)acc[v];
        const uint16_t kh = d2h_odd(acc[G]);
        a.k_hat[((int64_t)b * a.H + h) * kD + j] = kh;
        if constexpr (APPEND) khs[j] = kh;
    }
    if constexpr (APPEND) {
        __syncthreads();
        if (wave == 0)
            place_token(ap, b, h, 0, lane, khs[lane], khs[lane + 64],
                        u && ap.R == 0 ? wave_append_block(*u, ap, b, lane) : kTableBlock);
    }
}

template <int G, bool APPEND>
__global__ __launch_bounds__(kProjThreads) void k_project(ProjectArgs a, AppendArgs ap)
{
    project_unit<G, APPEND>(a, ap, blockIdx.x, blockIdx.y, nullptr);
}

// ---------------------------------------------------------------------------
// a paged step's projection, append and block-table update in one launch
// ---------------------------------------------------------------------------

// plane 0 / 1: key / value indices, 2 / 3: key / value values.  Blocks are
// [H][bs][row] per plane; row `skip` of every head is left alone (-1: none).
__device__ void copy_plane_skip(const AppendArgs &ap, int plane, int src, int dst, int skip)
{
    const SparseGeom &g = ap.geom;
    uint8_t *const base[4] = {ap.kidx, ap.vidx, ap.kval, ap.vval};
    const int entries = (plane & 1) ? g.ks_v : g.ks;
    const int64_t row_bytes = (int64_t)entries * (plane < 2 ? 1 : g.vbytes); // a power of two >= 8
    const int64_t bytes = (int64_t)g.H * g.bs * row_bytes;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 *s = (const u32x2 *)(base[plane] + (int64_t)src * bytes);
    u32x2 *d = (u32x2 *)(base[plane] + (int64_t)dst * bytes);
    for (int64_t j = threadIdx.x; j < bytes / 8; j += kProjThreads)
        if ((int)((j * 8 / row_bytes) % g.bs) != skip) d[j] = s[j];
}

// Workgroups 0 .. H B - 1: unit (h, b) = (i % H, i / H), projected and
// appended; workgroup H B writes the table entries; H B + 1 + 4 c + p copies
// plane p of copy c.
template <int G>
__global__ __launch_bounds__(kProjThreads) void k_project_paged(ProjectArgs a, AppendArgs ap, StepUpdateArgs u)
{
    const int units = a.H * a.B, i = blockIdx.x;
    if (i < units) {
        project_unit<G, true>(a, ap, i % a.H, i / a.H, &u);
    } else if (i == units) {
        for (int t = threadIdx.x; t < u.n_entries; t += kProjThreads) u.table[u.entry[t][0]] = u.entry[t][1];
    } else {
        const int c = (i - units - 1) / 4, plane = (i - units - 1) % 4;
        copy_plane_skip(ap, plane, u.copy[c][0], u.copy[c][1], u.copy[c][2]);
    }
}

template <bool APPEND>
static hipError_t launch_g(const ProjectArgs &a, const AppendArgs &ap, hipStream_t s)
{
    const dim3 grid(a.H, a.B), block(kProjThreads);
    switch (a.N_h / a.H) {
    case 1: hipLaunchKernelGGL((k_project<1, APPEND>), grid, block, 0, s, a, ap); break;
    case 2: hipLaunchKernelGGL((k_project<2, APPEND>), grid, block, 0, s, a, ap); break;
    case 4: hipLaunchKernelGGL((k_project<4, APPEND>), grid, block, 0, s, a, ap); break;
    case 8: hipLaunchKernelGGL((k_project<8, APPEND>), grid, block, 0, s, a, ap); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_project(const ProjectArgs &a, hipStream_t s) { return launch_g<false>(a, AppendArgs{}, s); }

hipError_t launch_project_append(const ProjectArgs &p, const AppendArgs &a, hipStream_t s)
{
    return launch_g<true>(p, a, s);
}

hipError_t launch_project_append_paged(const ProjectArgs &p, const AppendArgs &a, const StepUpdateArgs &u,
                                       hipStream_t s)
{
    const dim3 grid(p.H * p.B + 1 + 4 * u.n_copies), block(kProjThreads);
    switch (p.N_h / p.H) {
    case 1: hipLaunchKernelGGL(k_project_paged<1>, grid, block, 0, s, p, a, u); break;
    case 2: hipLaunchKernelGGL(k_project_paged<2>, grid, block, 0, s, p, a, u); break;
    case 4: hipLaunchKernelGGL(k_project_paged<4>, grid, block, 0, s, p, a, u); break;
    case 8: hipLaunchKernelGGL(k_project_paged<8>, grid, block, 0, s, p, a, u); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace swan
