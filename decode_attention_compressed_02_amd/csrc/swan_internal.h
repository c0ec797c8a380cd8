// swan_internal.h -- device helpers and launcher declarations shared by the
// HIP translation units of libswan (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swan.h"
#include "swan_measure.h"

namespace swan {

constexpr int kD = 128;          // head dimension (indices fit in 8 bits)
constexpr int kWave = 64;        // CDNA wavefront
constexpr int kCUs = 256;          // MI355X compute units (launch sizing only)
constexpr int kLdsPerCU = 160 * 1024;
constexpr int kMaxWaves = 1 << 20; // waves of one split pass (bounds the workspace)

// log2(e) / sqrt(128): scores are kept in base-2 units so softmax uses exp2
constexpr float kScoreScaleLog2 = 0.12751743074573063f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
// round to nearest even (the default mode of v_cvt_f16_f32)
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// fp16 bits of a double, rounded once to nearest even (IEEE 754 binary16:
// 10 stored significand bits, exponent bias 15, subnormal spacing 2^-24).
// Going through float first would round twice and can land one ulp off
// when the float lies on an fp16 midpoint.
__host__ __device__ inline uint16_t d2h(double x)
{
    const uint64_t bits = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    const int ex = (int)((bits >> 52) & 0x7FF);
    const uint64_t man = bits & ((1ull << 52) - 1);
    if (ex == 0x7FF) return sign | (man ? 0x7E00u : 0x7C00u); // NaN, infinity
    const int e = ex - 1023;                                   // x = 1.man * 2^e (normal doubles)
    if (e > 15) return sign | 0x7C00u;                         // >= 65536: overflow
    int shift;          // significand bits below the kept ones
    uint64_t sig;       // significand with its leading one
    uint32_t base;      // exponent field of the result before rounding
    if (e >= -14) {     // normal fp16
        sig = man;
        shift = 42;
        base = (uint32_t)(e + 15) << 10;
    } else {            // subnormal fp16 (or zero): units of 2^-24
        if (ex == 0 || e < -25) return sign; // below half the smallest subnormal
        sig = man | (1ull << 52);
        shift = 28 - e; // 43 .. 53
        base = 0;
    }
    const uint64_t kept = sig >> shift, rest = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    const uint32_t up = (rest > half || (rest == half && (kept & 1))) ? 1u : 0u;
    // a carry out of the significand steps the exponent (up to infinity)
    return sign | (uint16_t)(base + (uint32_t)kept + up);
}

// E4M3 bits of an fp16 value, rounded once to nearest even and saturating
// at +-448 (OCP E4M3: exponent bias 7, 3 fraction bits, subnormal spacing
// 2^-9, largest finite 448, code S.1111.111 NaN, no infinities).  Integer
// only: the fp16 significand is shifted to the E4M3 grid of its exponent.
__host__ __device__ inline uint8_t h2e4m3(uint16_t h)
{
    const uint32_t sign = (h >> 8) & 0x80u, mag = h & 0x7fffu;
    if (mag > 0x7c00u) return (uint8_t)(sign | 0x7fu); // NaN
    const uint32_t E = mag >> 10, M = mag & 0x3ffu;
    if (E >= 9) { // at least 2^-6: normal E4M3 (or beyond its range)
        uint32_t e = E - 8, sig = 1024u + M;            // 1.M with 10 fraction bits
        uint32_t kept = sig >> 7, rest = sig & 127u;    // keep 1 + 3 bits
        kept += (rest > 64u || (rest == 64u && (kept & 1u))) ? 1u : 0u;
        if (kept == 16u) { // carried into the next binade
            kept = 8u;
            ++e;
        }
        if (e > 15u || (e == 15u && kept == 15u)) return (uint8_t)(sign | 0x7eu); // past 448: saturate
        return (uint8_t)(sign | (e << 3) | (kept - 8u));
    }
    // below 2^-6: multiples of 2^-9, i.e. of 2^15 units of 2^-24
    const uint32_t v24 = E ? ((1024u + M) << (E - 1)) : M;
    uint32_t kept = v24 >> 15;
    const uint32_t rest = v24 & 0x7fffu;
    kept += (rest > 0x4000u || (rest == 0x4000u && (kept & 1u))) ? 1u : 0u; // 8 -> 2^-6, the smallest normal
    return (uint8_t)(sign | kept);
}

// Where the sparse rows of one (sequence, kv head) live.
struct SparseGeom {
    int H;          // kv heads
    int ks;         // entries per stored key row
    int ks_v;       // entries per stored value row (ks unless keys and values keep different counts)
    int n_cap;      // contiguous: rows per unit
    int bs;         // paged: rows per block (0 = contiguous)
    int max_blocks; // paged: block-table width
    int num_blocks; // paged: blocks in the pool
    int vbytes;     // bytes per stored value: 2 (fp16) or 1 (fp8 E4M3)
    const int32_t *bt;
};

// Row slot of sparse row r of unit (b, h), r below the unit's row
// capacity: the row starts at entry slot * ks of a key plane and slot * ks_v
// of a value plane.  Paged: -1 when the block-table entry is not a block of
// the pool (a caller error), so kernels skip the row instead of addressing
// outside the planes.
template <bool PAGED>
__device__ __forceinline__ int64_t row_slot(const SparseGeom &g, int b, int h, int r)
{
    if constexpr (PAGED) {
        const int blk = g.bt[(int64_t)b * g.max_blocks + r / g.bs];
        if (blk < 0 || blk >= g.num_blocks) return -1;
        return ((int64_t)blk * g.H + h) * g.bs + (r % g.bs);
    } else {
        return ((int64_t)b * g.H + h) * g.n_cap + r;
    }
}

__device__ __forceinline__ int64_t row_slot_rt(const SparseGeom &g, int b, int h, int r)
{
    return g.bs > 0 ? row_slot<true>(g, b, h, r) : row_slot<false>(g, b, h, r);
}

// Block of an appended row when the caller already knows it (a paged step
// whose table entries travel in the same launch): kTableBlock means "read the
// block table".
constexpr int kTableBlock = -0x7fffffff;
__device__ __forceinline__ int64_t append_row_slot(const SparseGeom &g, int b, int h, int r, int blk)
{
    if (blk == kTableBlock) return row_slot_rt(g, b, h, r);
    if (blk < 0 || blk >= g.num_blocks) return -1;
    return ((int64_t)blk * g.H + h) * g.bs + (r % g.bs);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane)); }

// Magnitude top-k of one 128-vector held by a full wave, two fp16 per lane
// (coordinate lane in `lo`, coordinate lane + 64 in `hi`).  Coordinates are
// ranked by (fp16 magnitude bits descending, index ascending); the k first
// are written to the row with ascending indices, values copied bit for bit
// (vbytes 2) or rounded to E4M3 (vbytes 1; the selection is still on the
// fp16 magnitudes), and entries k..ks-1 are zero padding.  Integer-only, so
// the selection is exact.  Must be called by all 64 lanes.
__device__ __forceinline__ void wave_prune_row(int lane, uint16_t lo, uint16_t hi, int k, int ks, uint8_t *idx_row,
                                               uint8_t *val_row, int vbytes)
{
    auto put = [&](int o, uint16_t v) {
        if (vbytes == 1)
            val_row[o] = h2e4m3(v);
        else
            ((uint16_t *)val_row)[o] = v;
    };
    const uint32_t mlo = lo & 0x7fffu, mhi = hi & 0x7fffu;
    // T = the k-th largest magnitude, found bit by bit from the top: the
    // largest T with at least k magnitudes >= T (ballots and popcounts only)
    uint32_t T = 0;
#pragma unroll
    for (int bit = 14; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        if (__popcll(__ballot(mlo >= c)) + __popcll(__ballot(mhi >= c)) >= k) T = c;
    }
    // rank of a coordinate = #(larger magnitudes) + #(equal magnitudes at
    // smaller indices); it is < k for every magnitude above T and for the
    // first k - #(above T) coordinates equal to T in index order (the lower
    // half's indices precede the upper half's)
    const int need = k - (__popcll(__ballot(mlo > T)) + __popcll(__ballot(mhi > T)));
    const uint64_t eq_lo = __ballot(mlo == T), eq_hi = __ballot(mhi == T);
    const uint64_t below = lanemask_lt(lane);
    const bool keep_lo = mlo > T || (mlo == T && __popcll(eq_lo & below) < need);
    const bool keep_hi = mhi > T || (mhi == T && __popcll(eq_lo) + __popcll(eq_hi & below) < need);
    const uint64_t blo = __ballot(keep_lo), bhi = __ballot(keep_hi);
    if (keep_lo) {
        const int o = __popcll(blo & below);
        idx_row[o] = (uint8_t)lane;
        put(o, lo);
    }
    if (keep_hi) {
        const int o = __popcll(blo) + __popcll(bhi & below);
        idx_row[o] = (uint8_t)(lane + 64);
        put(o, hi);
    }
    if (lane < ks - k) {
        idx_row[k + lane] = 0;
        put(k + lane, 0);
    }
}

// ---- launchers (defined in the .hip files; no validation, grids checked by caller)

struct ProjectArgs {
    int B, N_h, H;
    const float *q, *k;
    const int32_t *pos;
    const float *P; // [layers][H][128][128]; sequence b uses layer b / Bl
    float base;
    float *q_hat;
    uint16_t *k_hat;
    int Bl; // sequences per layer (B when the batch is one layer)
};
hipError_t launch_project(const ProjectArgs &a, hipStream_t s);

struct AppendArgs {
    int B, H, R, k, k_v; // kept key and value coordinates
    SparseGeom geom;
    uint8_t *kidx, *vidx;
    uint8_t *kval, *vval; // value planes, geom.vbytes bytes per entry
    uint16_t *kbuf, *vbuf;
    const int32_t *pos;
    const uint16_t *k_hat;
    const float *v_hat;
};
hipError_t launch_append(const AppendArgs &a, hipStream_t s);

// Append of one token to unit (b, h) by one wave, in two parts: `wave` 0
// handles the key, 1 the value; (lo, hi) are the token's fp16 coordinates
// lane and lane + 64.  evict_token prunes the token leaving the circular
// buffer (slot = position mod R, holding token pos - R) into its sparse row;
// it needs nothing of the new token, so it may run before the new key is
// known.  place_token then writes the new token into that slot; with R = 0 it
// prunes the new token straight into row pos.  Inactive sequences (pos < 0)
// append nothing.  The two parts must run in this order (the slot is read
// before it is overwritten).
__device__ inline void evict_token(const AppendArgs &a, int b, int h, int wave, int lane, int blk = kTableBlock)
{
    const int p = a.pos[b];
    if (p < a.R || a.R == 0) return; // also p < 0
    const int64_t u = (int64_t)b * a.H + h;
    const uint16_t *buf = (wave == 0 ? a.kbuf : a.vbuf) + (u * a.R + p % a.R) * kD;
    const uint16_t olo = buf[lane], ohi = buf[lane + 64];
    const int r = p - a.R;
    const int row_cap = a.geom.bs > 0 ? a.geom.max_blocks * a.geom.bs : a.geom.n_cap;
    const int64_t slot = r < row_cap ? append_row_slot(a.geom, b, h, r, blk) : -1;
    if (slot < 0) return;
    const int vb = a.geom.vbytes, kk = wave == 0 ? a.k : a.k_v, ks = wave == 0 ? a.geom.ks : a.geom.ks_v;
    wave_prune_row(lane, olo, ohi, kk, ks, (wave == 0 ? a.kidx : a.vidx) + slot * ks,
                   (wave == 0 ? a.kval : a.vval) + slot * ks * vb, vb);
}

__device__ inline void place_token(const AppendArgs &a, int b, int h, int wave, int lane, uint16_t lo, uint16_t hi,
                                   int blk = kTableBlock)
{
    const int p = a.pos[b];
    if (p < 0) return;
    const int64_t u = (int64_t)b * a.H + h;
    if (a.R == 0) {
        const int row_cap = a.geom.bs > 0 ? a.geom.max_blocks * a.geom.bs : a.geom.n_cap;
        const int64_t slot = p < row_cap ? append_row_slot(a.geom, b, h, p, blk) : -1;
        if (slot < 0) return;
        const int vb = a.geom.vbytes, kk = wave == 0 ? a.k : a.k_v, ks = wave == 0 ? a.geom.ks : a.geom.ks_v;
        wave_prune_row(lane, lo, hi, kk, ks, (wave == 0 ? a.kidx : a.vidx) + slot * ks,
                       (wave == 0 ? a.kval : a.vval) + slot * ks * vb, vb);
        return;
    }
    uint16_t *buf = (wave == 0 ? a.kbuf : a.vbuf) + (u * a.R + p % a.R) * kD;
    buf[lane] = lo;
    buf[lane + 64] = hi;
}

__device__ inline void append_token(const AppendArgs &a, int b, int h, int wave, int lane, uint16_t lo, uint16_t hi,
                                    int blk = kTableBlock)
{
    evict_token(a, b, h, wave, lane, blk);
    place_token(a, b, h, wave, lane, lo, hi, blk);
}

// projection and append of a step in one launch (the append waits for the
// unit's new key inside the workgroup, not for the whole grid)
hipError_t launch_project_append(const ProjectArgs &p, const AppendArgs &a, hipStream_t s);

// A paged step's block-table writes and copy-on-write copies carried by value
// into the projection/append launch.  The appends take their rows' blocks
// from these entries (so they never read a table entry the same launch
// writes), and copy i skips row skip of every head of its destination: the
// row this launch's append writes there.  No two workgroups then touch the
// same bytes, so the launch needs no ordering inside it.
constexpr int kFusedEntries = 192, kFusedCopies = 32;
struct StepUpdateArgs {
    int n_entries, n_copies;
    int32_t *table;
    int32_t entry[kFusedEntries][2]; // (b * max_blocks + j, block id); slots distinct
    int32_t copy[kFusedCopies][3];   // (src, dst, skip row or -1)
};
hipError_t launch_project_append_paged(const ProjectArgs &p, const AppendArgs &a, const StepUpdateArgs &u,
                                       hipStream_t s);

// Shape of the sparse stream in the split kernel for GQA group G, stored key
// rows of KS entries and value rows of KSV entries (KSmax the wider).  TPI
// rows (tokens) are in flight per wave iteration, one per accumulator slot,
// and lane l works on row slot l % TPI; the 64 / TPI lanes of a row each load
// E = KS TPI / 64 consecutive key entries and EV = KSV TPI / 64 value entries.
// A 128-bit LDS access is served in 16-lane phases over 16 bank quads, and
// the accumulators are laid out as acc[c][slot][g], so with 16 slots the 16
// lanes of a phase always hit 16 different quads: the value scatter runs
// without bank conflicts whatever the indices are.  G = 8 keeps 8 slots (LDS
// size).  Rows of 64 or more entries also use 8 slots: half the accumulator
// LDS lets two waves share a SIMD, and with 8 or more entries per lane the
// row sums stay cheap; measured faster than 16 slots at one wave per SIMD.
__host__ __device__ constexpr int split_slots(int G, int KSmax) { return (G <= 4 && KSmax <= 32) ? 16 : 8; }
// resident waves per SIMD the split kernel is compiled for (register budget:
// 256 registers a lane at two waves; wider rows and g = 8 need more)
__host__ __device__ constexpr int split_waves_per_simd(int G, int KSmax) { return (G <= 4 && KSmax == 64) ? 2 : 1; }
// entries per lane of a row of KS entries (1..16 for KS in 8..128)
__host__ __device__ constexpr int split_entries(int G, int KS, int KSmax) { return KS * split_slots(G, KSmax) / 64; }
// LDS bytes of one split workgroup: the scaled queries plus the accumulator slots
__host__ __device__ constexpr int split_lds_bytes(int G, int KSmax)
{
    return 4 * kD * G * (1 + split_slots(G, KSmax));
}
// split waves resident on one CU: the LDS footprint and, for g >= 4, the
// register budget above (g <= 2 fits at least two waves per SIMD)
__host__ __device__ constexpr int split_waves_per_cu(int G, int KSmax)
{
    const int by_lds = kLdsPerCU / split_lds_bytes(G, KSmax), by_regs = G >= 4 ? 4 * split_waves_per_simd(G, KSmax) : 8;
    const int w = by_lds < by_regs ? by_lds : by_regs;
    return w < 1 ? 1 : w;
}

// ---- work plan of the decode split pass
// Each unit (sequence b, kv head h) is a run of work rows in one virtual
// sequence over all units, b-major then h: one per sparse row plus, per
// buffered token, its bytes relative to a sparse row (a buffered token
// streams 2 x 256 bytes, a sparse row (1 + value bytes) (KS + KSV)).  The T work rows of the
// batch are cut into V nearly equal ranges, wave w taking [w T / V,
// (w + 1) T / V) (rounded down), so every wave streams about the same bytes
// whatever the mix of lengths; when V is a multiple of the unit count and
// the units are equally long, every range lies inside one unit.  A piece
// [lo, hi) of a unit's work rows covers the same fraction of its sparse rows
// (in whole ring slots of kSparseQuantum rows) and of its buffered tokens.
// A wave may cover the end of one unit and the start of the next, one
// partial per piece: the piece of unit u in wave w writes partial w + u
// (pieces in work-row order step w, u or both by one, so the index is unique
// and below V + B H).
constexpr int kSparseQuantum = 16; // a multiple of the rows per ring slot
constexpr int kMinWaveRows = 64;

// work rows of buffered tokens [0, f) when a stored sparse row (key and
// value planes) is row_bytes bytes
__host__ __device__ inline int64_t dense_work(int64_t f, int row_bytes) { return (f * 512 + row_bytes - 1) / row_bytes; }
__host__ __device__ constexpr int sparse_row_bytes(int ks, int ks_v, int vbytes) { return (1 + vbytes) * (ks + ks_v); }

struct UnitWork {
    int64_t n, f, len; // sparse rows, buffered tokens, work rows
};
__host__ __device__ inline UnitWork unit_work(int32_t pos, int R, int64_t row_cap, int row_bytes)
{
    const int64_t ctx = (int64_t)pos + 1; // <= 0: inactive sequence
    UnitWork u;
    u.n = ctx > R ? ctx - R : 0;
    if (u.n > row_cap) u.n = row_cap;
    u.f = ctx <= 0 ? 0 : (ctx < R ? ctx : R);
    u.len = u.n + dense_work(u.f, row_bytes);
    return u;
}
// first sparse row of the piece starting at work row x of the unit (0 <= x
// <= len): a multiple of kSparseQuantum, or n at the end
__host__ __device__ inline int64_t sparse_split(int64_t x, const UnitWork &u)
{
    if (x >= u.len) return u.n;
    const int64_t r = x * ((u.n + kSparseQuantum - 1) / kSparseQuantum) / u.len * kSparseQuantum;
    return r < u.n ? r : u.n;
}
// first buffered token of the piece starting at work row x
__host__ __device__ inline int64_t dense_split(int64_t x, const UnitWork &u)
{
    return x >= u.len ? u.f : (x * u.f + u.len - 1) / u.len;
}
// waves V that take part for a batch of T work rows and a grid of W waves
__host__ __device__ inline int64_t active_waves(int64_t T, int W, int split_tokens)
{
    int64_t v = split_tokens > 0 ? (T + split_tokens - 1) / split_tokens : T / kMinWaveRows;
    if (v > W) v = W;
    return v < 1 ? 1 : v;
}

struct SplitArgs {
    int B, N_h, H, R;
    int W;            // waves of the split pass (the grid)
    int split_tokens; // about this many work rows per wave; 0: spread the batch over W waves
    int k, k_v;       // kept key and value entries per row; the rest of a stored row is padding
    int row_cap;      // sparse rows addressable per unit
    SparseGeom geom;
    const int32_t *pos;
    const float *q_hat;
    const uint8_t *kidx, *vidx;
    const uint8_t *kval, *vval; // value planes, geom.vbytes bytes per entry
    const uint16_t *kbuf, *vbuf;
    float *part_o;  // [W + B H][g][128]
    float *part_ml; // [W + B H][g][2]
};
hipError_t launch_split(const SplitArgs &a, int g, hipStream_t s);
hipError_t launch_split_g1(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g2(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g4(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g8(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g1_paged(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g2_paged(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g4_paged(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g8_paged(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g1_paged_rows(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g2_paged_rows(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g4_paged_rows(const SplitArgs &a, hipStream_t s);
hipError_t launch_split_g8_paged_rows(const SplitArgs &a, hipStream_t s);
// Paged pools whose blocks hold a power-of-two multiple of the split pass's
// ring-slot rows read each slot through one block (its id through the scalar
// cache); other block sizes look the block up per row (the _rows kernels).
inline bool paged_slot_blocks(int G, const SparseGeom &g)
{
    const int tpi = split_slots(G, g.ks > g.ks_v ? g.ks : g.ks_v);
    return g.bs > 0 && g.bs % tpi == 0 && (g.bs & (g.bs - 1)) == 0;
}

struct ReduceArgs {
    int B, N_h, H, R, W, split_tokens, row_bytes, row_cap;
    const int32_t *pos;
    const float *part_o, *part_ml;
    float *o_hat;
};
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);

struct PrefillArgs {
    int B, H, R, k, k_v;
    int64_t T_stride;
    int max_len;
    SparseGeom geom;
    uint8_t *kidx, *vidx;
    uint8_t *kval, *vval; // value planes, geom.vbytes bytes per entry
    uint16_t *kbuf, *vbuf;
    const int32_t *len;
    const float *k_raw, *v_hat, *P; // P: [layers][H][128][128]; sequence b uses layer b / Bl
    float base;
    int Bl; // sequences per layer
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

struct CopyBlocksArgs {
    int count, num_blocks;
    int64_t block_bytes_kidx, block_bytes_vidx; // bytes of one block of the key / value index plane
    int vbytes;                                 // value planes: vbytes times their index plane
    uint8_t *kidx, *vidx;
    uint8_t *kval, *vval;
    const int32_t *src, *dst;
};
hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t s);

// Block-table writes and copy-on-write copies of a paged step carried in the
// launch's own arguments (no host-to-device copy on the stream): workgroup 0
// writes the table entries, workgroup 1 + 4 i + p copies plane p of copy i.
constexpr int kUpdateEntries = 192, kUpdateCopies = 32; // per launch
struct PagedUpdateArgs {
    int n_entries, n_copies, num_blocks;
    int64_t block_bytes_kidx, block_bytes_vidx;
    int vbytes;
    uint8_t *kidx, *vidx;
    uint8_t *kval, *vval;
    int32_t *table;
    int32_t entry[kUpdateEntries][2]; // (b * max_blocks + j, block id)
    int32_t copy[kUpdateCopies][2];   // (src, dst)
};
hipError_t launch_paged_update(const PagedUpdateArgs &a, hipStream_t s);

// streaming read of a buffer (swan_measure.h): waves one-wave workgroups,
// bytes a multiple of 16, sink of waves * 64 words
hipError_t launch_stream_read(const void *buf, int64_t bytes, int waves, uint32_t *sink, hipStream_t s);

} // namespace swan
