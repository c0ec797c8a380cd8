// split_kernel.h -- hybrid decode attention (SWAN page, hybrid-cache
// paragraphs and Appendix A.2, steps 2-4): scores of the rotated query against the sparse history (an
// indexed gather of q_hat) and the dense buffer, one softmax over both, and
// the output accumulated from sparse values (scatter-add at the stored
// indices) and dense values.
//
// Pass 1 (k_split): wavefronts over nearly equal ranges of the batch's work
// rows (the work plan in swan_internal.h).  A wave serves all g query heads of
// the GQA group, so every row streamed from HBM is used g times.  For each
// piece of a (sequence, kv head) in its range it keeps an online softmax
// (running max m, running sum l) over the piece's sparse rows and buffered
// tokens and writes (m, l, unnormalised output) per query head.
//
// Sparse stream: a stored row is KS entries (uint8 index, fp16 or fp8 value).  A
// lane loads E consecutive entries of one row from each of the four planes
// (K index, K value, V index, V value), KS / E lanes share a row and TPI =
// 64 E / KS rows are in flight per wave iteration, so each wave load
// instruction reads one contiguous span of a plane.  Loads run D iterations
// ahead of the arithmetic (a register ring), which keeps enough bytes in
// flight per wave to cover HBM latency.
//
// LDS holds the scaled q_hat of the group as qs[c][g] (one 16-byte gather per
// stored key index for g = 4) and TPI private copies of the output
// accumulator, one per row slot of an iteration, interleaved as
// acc[c][slot][g].  The indices of one row are distinct and different slots
// write different copies, so the value scatter is a plain read-modify-write
// of 16 bytes per entry with no two lanes of an instruction touching the same
// address: no LDS atomics (floating-point LDS atomics are an order of
// magnitude slower than plain accesses on gfx950).  Lane l serves slot
// l % TPI; with TPI = 16 the 16 lanes of each 128-bit LDS phase fall in 16
// different bank quads, so the scatter has no bank conflicts.  (With TPI = 8
// the two lanes of a slot in a phase can meet in a quad; a padded layout that
// avoids it needs 2 KB more LDS per wave and measured slower.)  Partial sums
// over the lanes of a row use DPP and the gfx950 permlane swaps, not LDS.
//
// Scores are in base-2 units (q_hat pre-scaled by log2(e)/sqrt(d_h)).  The
// running max is raised only when a score exceeds it by more than
// kRescaleSlack, so the accumulator rescale (a pass over LDS) is rare; weights
// stay below 2^kRescaleSlack.
//
// Buffered tokens: 16 lanes per token (8 coordinates each), 4 tokens per
// iteration, output accumulated in registers and folded into accumulator
// copy 0 before the sparse rows start.
//
// Pass 2 (k_reduce, decode.hip): one workgroup per (query head, sequence)
// merges the partials of the unit's pieces with log-sum-exp weights.
#pragma once

#include "swan_internal.h"

namespace swan {

constexpr float kRescaleSlack = 8.0f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// lane-group reductions and small LDS vector accessors
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of L consecutive lanes; every lane of a group gets
// the group's sum.  quad_perm [1,0,3,2] and [2,3,0,1] are xor 1 and xor 2;
// once each quad holds its sum, the half-row mirror pairs the two quads of
// an 8-lane group and the row mirror pairs the two halves of a 16-lane row.
template <int L>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (L >= 2) x += dpp<0xB1>(x);
    if constexpr (L >= 4) x += dpp<0x4E>(x);
    if constexpr (L >= 8) x += dpp<0x141>(x);
    if constexpr (L >= 16) x += dpp<0x140>(x);
    if constexpr (L >= 32) x += __shfl_xor(x, 16);
    if constexpr (L >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Sum over the lanes that share lane % TPI (TPI = 8 or 16): row_ror:8 pairs
// lanes 8 apart inside a 16-lane row, the permlane swaps pair rows 16 and 32
// lanes apart.  Every lane of a group adds the same operands in the same
// order, so all of them hold the bit-identical sum.
//
// __builtin_bit_cast applied directly to an element of the returned vector
// reads element 0 whatever the index, so the elements are copied out first.
__device__ __forceinline__ float swap_sum16(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned a = r[0], b = r[1];
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float swap_sum32(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned a = r[0], b = r[1];
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
template <int TPI>
__device__ __forceinline__ float slot_sum(float x)
{
    static_assert(TPI == 8 || TPI == 16, "slot_sum covers 8 or 16 slots");
    if constexpr (TPI == 8) x += dpp<0x128>(x);
    return swap_sum32(swap_sum16(x));
}

// Transposed row sums for g = 4 and 16 row slots.  Lane l holds partial
// scores s0..s3 (one per query head) of row slot l % 16; the four lanes of a
// slot sit in the four 16-lane rows.  Three swaps leave every lane with the
// full score of one head of its slot: row 0 -> head 0, row 1 -> head 2,
// row 2 -> head 1, row 3 -> head 3 (transposed_head).  The swap pairs
// (s0, s2) and (s1, s3) so that each half of a row pair keeps what the other
// half sends: no selects and no copies.
__device__ __forceinline__ int transposed_head(int lane)
{
    const int row = lane >> 4;
    return ((row & 1) << 1) | (row >> 1);
}
__device__ __forceinline__ float swap16_add(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    const unsigned x = r[0], y = r[1];
    return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float swap32_add(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    const unsigned x = r[0], y = r[1];
    return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float transposed_sum4(float s0, float s1, float s2, float s3)
{
    // even rows: s0 of the row pair, odd rows: s2; likewise (s1, s3)
    const float u = swap16_add(s0, s2), v = swap16_add(s1, s3);
    // lower half keeps u (heads 0 / 2), upper half keeps v (heads 1 / 3)
    return swap32_add(u, v);
}
// Inverse of the transposition: every lane gets the values of heads 0..3 of
// its row slot from the four lanes that hold them.
__device__ __forceinline__ void transposed_broadcast4(float x, float (&o)[4])
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false); // (row 2k, row 2k+1)
    const unsigned a0 = a[0], a1 = a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(a0, a0, false, false); // heads 0, 1
    const auto c = __builtin_amdgcn_permlane32_swap(a1, a1, false, false); // heads 2, 3
    const unsigned b0 = b[0], b1 = b[1], c0 = c[0], c1 = c[1];
    o[0] = __builtin_bit_cast(float, b0);
    o[1] = __builtin_bit_cast(float, b1);
    o[2] = __builtin_bit_cast(float, c0);
    o[3] = __builtin_bit_cast(float, c1);
}
// max over the 16 lanes of a row (every lane gets it)
__device__ __forceinline__ float row_max16(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
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

// value of lane l (wave-uniform l), in scalar registers
__device__ __forceinline__ int64_t lane_value(int64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l), hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// inclusive prefix sum over the lanes of the wave
__device__ __forceinline__ int64_t wave_scan(int64_t v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// work rows of the units of sequences [0, B) (per kv head), summed over the
// lanes of a wave or a block's waves alike
__device__ __forceinline__ int64_t seq_work(const int32_t *pos, int b, int R, int64_t row_cap, int row_bytes)
{
    return unit_work(pos[b], R, row_cap, row_bytes).len;
}

// G consecutive floats of LDS at p (16-byte aligned for G >= 4)
template <int G>
__device__ __forceinline__ void lds_get(const float *p, float (&v)[G])
{
    if constexpr (G == 1) {
        v[0] = p[0];
    } else if constexpr (G == 2) {
        const f32x2 t = *(const f32x2 *)p;
        v[0] = t.x;
        v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < G; i += 4) {
            const f32x4 t = *(const f32x4 *)(p + i);
            v[i] = t.x;
            v[i + 1] = t.y;
            v[i + 2] = t.z;
            v[i + 3] = t.w;
        }
    }
}

template <int G>
__device__ __forceinline__ void lds_put(float *p, const float (&v)[G])
{
    if constexpr (G == 1) {
        p[0] = v[0];
    } else if constexpr (G == 2) {
        *(f32x2 *)p = (f32x2){v[0], v[1]};
    } else {
#pragma unroll
        for (int i = 0; i < G; i += 4) *(f32x4 *)(p + i) = (f32x4){v[i], v[i + 1], v[i + 2], v[i + 3]};
    }
}

// ---------------------------------------------------------------------------
// streaming loads of NB bytes into 32-bit words (non-temporal: every byte of
// the history is read once per step)
// ---------------------------------------------------------------------------

template <int NB>
struct Words {
    static constexpr int N = NB < 4 ? 1 : NB / 4;
    uint32_t w[N];
};

template <int NB>
__device__ __forceinline__ void load_words(const void *p, Words<NB> &o)
{
    if constexpr (NB == 1) {
        o.w[0] = __builtin_nontemporal_load((const uint8_t *)p);
    } else if constexpr (NB == 2) {
        o.w[0] = __builtin_nontemporal_load((const uint16_t *)p);
    } else if constexpr (NB == 4) {
        o.w[0] = __builtin_nontemporal_load((const uint32_t *)p);
    } else if constexpr (NB == 8) {
        const u32x2 t = __builtin_nontemporal_load((const u32x2 *)p);
        o.w[0] = t.x;
        o.w[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const u32x4 t = __builtin_nontemporal_load((const u32x4 *)p + i);
            o.w[4 * i] = t.x;
            o.w[4 * i + 1] = t.y;
            o.w[4 * i + 2] = t.z;
            o.w[4 * i + 3] = t.w;
        }
    }
}

// NB bytes at byte offset off of a buffer resource (raw, non-temporal).
// Offsets at or past the resource's size read zeros without touching memory.
template <int NB>
__device__ __forceinline__ void buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t off, Words<NB> &o)
{
    constexpr int kNT = 2; // cache policy: non-temporal
    if constexpr (NB == 1) {
        o.w[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kNT);
    } else if constexpr (NB == 2) {
        o.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNT);
    } else if constexpr (NB == 4) {
        o.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT);
    } else if constexpr (NB == 8) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT);
        o.w[0] = t.x;
        o.w[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, kNT);
            o.w[4 * i] = t.x;
            o.w[4 * i + 1] = t.y;
            o.w[4 * i + 2] = t.z;
            o.w[4 * i + 3] = t.w;
        }
    }
}

// raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int NB>
__device__ __forceinline__ int byte_at(const Words<NB> &o, int e)
{
    return (int)((o.w[e >> 2] >> ((e & 3) * 8)) & 0xffu);
}

// (index byte e of the row) * 256 + slot_off, for slot_off < 256: one
// v_perm_b32 puts the index byte in byte 1 and slot_off in byte 0 (bytes 2-3
// zero).  With acc[c][16 slots][4 heads] of fp32, entry c of slot s sits at
// byte c * 256 + s * 16.
template <int NB>
__device__ __forceinline__ uint32_t acc_offset_256(const Words<NB> &o, int e, uint32_t slot_off)
{
    const uint32_t sel = 0x0c0c0000u | ((uint32_t)(4 + (e & 3)) << 8);
    return __builtin_amdgcn_perm(o.w[e >> 2], slot_off, sel);
}

// Value e of a row slice: fp16 (VB = 2 bytes) or fp8 E4M3 (VB = 1; the
// gfx950 conversion decodes the OCP E4M3 encoding exactly).  e is a
// compile-time constant after unrolling, so the byte select folds.
template <int VB, int NB>
__device__ __forceinline__ float value_at(const Words<NB> &o, int e)
{
    if constexpr (VB == 2) {
        return h2f((uint16_t)(o.w[e >> 1] >> ((e & 1) * 16)));
    } else {
        const uint32_t w = o.w[e >> 2];
        switch (e & 3) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
        }
    }
}

// E entries of one sparse row: the key planes and the value planes are
// separate ring slots (consumed in different phases); VB bytes per value
template <int E, int VB>
struct KSlot {
    Words<E> ki;
    Words<VB * E> kv;
    bool ok; // the row's block-table entry is a block of the pool
};
template <int E, int VB>
struct VSlot {
    Words<E> vi;
    Words<VB * E> vv;
};

// 2^x with the hardware instruction: arguments are <= kRescaleSlack, and
// results that would be denormal (x < -126) only ever weigh a token that is
// 2^-126 of the running max, so flushing them to zero is harmless
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// running-max value meaning "no score yet": finite, so exp2(-inf - kNoScore)
// is 0 rather than NaN, and far below any real score
constexpr float kNoScore = -1e30f;

// sched_barrier mask: ALU, transcendental and LDS instructions may move
// across, global loads may not (keeps ring loads in issue order)
constexpr int kKeepLoadOrder = 0x1 | 0x2 | 0x4 | 0x8 | 0x80 | 0x100 | 0x200 | 0x400;

// ---------------------------------------------------------------------------
// pass 1
// ---------------------------------------------------------------------------

// Ring depth of the sparse stream: about SWAN_INFLIGHT_BYTES per lane in
// flight (slice_bytes: a lane's slice of a row in the four planes), between 2
// and 8 slots.
#ifndef SWAN_INFLIGHT_BYTES
#define SWAN_INFLIGHT_BYTES 192
#endif
__host__ __device__ constexpr int split_depth(int slice_bytes)
{
    const int d = (SWAN_INFLIGHT_BYTES + slice_bytes - 1) / slice_bytes;
    return d < 2 ? 2 : (d > 8 ? 8 : d);
}

// SLOTS (paged pools only): every ring slot of TPI rows lies in one block
// (the block size is a power-of-two multiple of TPI, paged_slot_blocks);
// otherwise paged rows are looked up one at a time
template <int G, int KS, int KSV, bool PAGED, bool PAD, int VB, bool SLOTS>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(split_waves_per_simd(G, KS > KSV ? KS : KSV)))) void k_split(SplitArgs a)
{
    constexpr int KSM = KS > KSV ? KS : KSV;
    constexpr int TPI = split_slots(G, KSM); // rows per iteration = accumulator copies
    constexpr int LPT = kWave / TPI;         // lanes per row
    constexpr int E = split_entries(G, KS, KSM), EV = split_entries(G, KSV, KSM); // key / value entries a lane
    constexpr int kRowBytes = sparse_row_bytes(KS, KSV, VB);
    // fp8 values and narrower planes: the same bytes in flight in more slots,
    // except where the register budget of two waves per SIMD has no room for
    // them (there the depth is that of fp16 rows of the wider width)
    constexpr bool kTwoWaves = split_waves_per_simd(G, KSM) == 2;
    constexpr int D = split_depth(kTwoWaves ? 3 * 2 * (E > EV ? E : EV) : (1 + VB) * (E + EV));
    constexpr int CS = TPI * G; // accumulator floats per coordinate
    constexpr int NACC = kD * CS;
    static_assert(LPT * E == KS && LPT * EV == KSV && E >= 1 && EV >= 1 && E <= 16 && EV <= 16, "bad split shape");
    static_assert(split_lds_bytes(G, KSM) == 4 * (kD * G + NACC), "host and device disagree on LDS size");
    // g = 4 keeps sparse scores transposed, one (row slot, head) per lane (with
    // 8 row slots each pair sits in two lanes); otherwise every lane of a row
    // slot holds all g scores
    constexpr bool kT = (G == 4 && (TPI == 16 || TPI == 8));

    __shared__ __attribute__((aligned(16))) float qs[kD * G];
    __shared__ __attribute__((aligned(16))) float acc[NACC];

    const int lane = threadIdx.x;
    const int64_t w = blockIdx.x;

    // ---- this wave's work rows [x0, x1) of the batch.  Lane l holds
    // sequence base + l; the first 64 sequences stay in registers for the
    // search below (one pass when B <= 64).
    const int32_t pos0 = lane < a.B ? a.pos[lane] : -1;
    const int64_t len0 = lane < a.B ? unit_work(pos0, a.R, a.row_cap, kRowBytes).len * a.H : 0;
    const int64_t end0 = wave_scan(len0);
    int64_t total = lane_value(end0, kWave - 1);
    for (int base = kWave; base < a.B; base += kWave) {
        const int bb = base + lane;
        total += lane_value(wave_scan(bb < a.B ? seq_work(a.pos, bb, a.R, a.row_cap, kRowBytes) * a.H : 0), kWave - 1);
    }
    const int64_t V = active_waves(total, a.W, a.split_tokens);
    if (w >= V) return;
    const int64_t x0 = w * total / V, x1 = (w + 1) * total / V;
    if (x0 >= x1) return;
    // first sequence whose units reach past x0, and the work row they start at
    int b = 0;
    int64_t P = 0;
    {
        const uint64_t hit = __ballot(lane < a.B && end0 > x0);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            b = l;
            P = lane_value(end0 - len0, l);
        } else {
            int64_t run = lane_value(end0, kWave - 1);
            for (int base = kWave; base < a.B; base += kWave) {
                const int bb = base + lane;
                const int64_t len = bb < a.B ? seq_work(a.pos, bb, a.R, a.row_cap, kRowBytes) * a.H : 0;
                const int64_t end = run + wave_scan(len);
                const uint64_t hit2 = __ballot(bb < a.B && end > x0);
                if (hit2) {
                    const int l = __builtin_ctzll(hit2);
                    b = base + l;
                    P = lane_value(end - len, l);
                    break;
                }
                run = lane_value(end, kWave - 1);
            }
        }
    }
    for (; b < a.B && P < x1; ++b) {
        const int32_t pb = b < kWave ? __builtin_amdgcn_readlane(pos0, b) : __builtin_amdgcn_readfirstlane(a.pos[b]);
        const UnitWork uw = unit_work(pb, a.R, a.row_cap, kRowBytes);
        for (int h = (uw.len > 0 && x0 > P) ? (int)((x0 - P) / uw.len) : 0;
             uw.len > 0 && h < a.H && P + h * uw.len < x1; ++h) {
            // the piece [lo, hi) of unit (b, h): sparse rows [t0, t1) and buffered tokens [d0, d1)
            const int64_t us = P + h * uw.len, lo = max(x0, us) - us, hi = min(x1, us + uw.len) - us;
            const int t0 = (int)sparse_split(lo, uw), t1 = (int)sparse_split(hi, uw);
            const int d0 = (int)dense_split(lo, uw), d1 = (int)dense_split(hi, uw);
            const int64_t piece = (int64_t)w + (int64_t)b * a.H + h;

            const float *qsrc = a.q_hat + ((int64_t)b * a.N_h + h * G) * kD;
            {
                float qv[2 * G]; // all loads first, then the LDS writes
#pragma unroll
                for (int j = 0; j < 2 * G; ++j) qv[j] = qsrc[lane + j * kWave];
#pragma unroll
                for (int j = 0; j < 2 * G; ++j) {
                    const int i = lane + j * kWave, hh = i / kD, c = i % kD;
                    qs[c * G + hh] = qv[j] * kScoreScaleLog2;
                }
            }
            for (int i = lane * 4; i < NACC; i += kWave * 4) *(f32x4 *)(acc + i) = (f32x4){0.f, 0.f, 0.f, 0.f};
            __syncthreads();

            // Running max per head, kept finite (kNoScore) so that exp2(s - m) of a
            // masked score (-inf) is 0 without a NaN guard; ls counts the sparse
            // weights once per lane of a row (divided by LPT at the end), ld the
            // buffered weights once per token.
            float m[G], ls[G], ld[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                m[hh] = kNoScore;
                ls[hh] = 0.f;
                ld[hh] = 0.f;
            }

            // ---- buffered tokens [d0, d1)
            if (d0 < d1) {
                constexpr int DD = 4;
                const int tl = lane >> 4, c0 = (lane & 15) * 8;
                float qr[8][G], ar[8][G];
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        qr[i][hh] = qs[(c0 + i) * G + hh];
                        ar[i][hh] = 0.f;
                    }
                const int64_t ub = ((int64_t)b * a.H + h) * a.R * kD + c0;
                u32x4 kst[DD], vst[DD];
                auto dload = [&](int t, u32x4 &kk, u32x4 &vv) {
                    const int tok = min(t + tl, d1 - 1);
                    kk = __builtin_nontemporal_load((const u32x4 *)(a.kbuf + ub + (int64_t)tok * kD));
                    vv = __builtin_nontemporal_load((const u32x4 *)(a.vbuf + ub + (int64_t)tok * kD));
                };
#pragma unroll
                for (int d = 0; d < DD; ++d) {
                    dload(d0 + 4 * d, kst[d], vst[d]);
                    __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                }
                // steps past d1 run fully masked; each ring slot is consumed before
                // it is reloaded so the loop carries no register copies
                for (int tb = d0; tb < d1; tb += 4 * DD) {
#pragma unroll
                    for (int d = 0; d < DD; ++d) {
                        const int t = tb + 4 * d;
                        const half8 kh = __builtin_bit_cast(half8, kst[d]), vh = __builtin_bit_cast(half8, vst[d]);
                        const bool valid = t + tl < d1;
                        float s[G], dm = -INFINITY;
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) {
                            s[hh] = 0.f;
#pragma unroll
                            for (int i = 0; i < 8; ++i) s[hh] = fmaf(qr[i][hh], (float)kh[i], s[hh]);
                            const float gs = group_sum<16>(s[hh]); // all lanes take part in the permutes
                            s[hh] = valid ? gs : -INFINITY;
                            dm = fmaxf(dm, s[hh] - m[hh]);
                        }
                        if (__any(dm > kRescaleSlack)) { // wave-uniform
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) {
                                const float mn = fmaxf(m[hh], wave_max(s[hh]));
                                const float f = fast_exp2(m[hh] - mn);
                                m[hh] = mn;
                                ld[hh] *= f;
#pragma unroll
                                for (int i = 0; i < 8; ++i) ar[i][hh] *= f;
                            }
                        }
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) {
                            const float w = fast_exp2(s[hh] - m[hh]);
                            if ((lane & 15) == 0) ld[hh] += w;
#pragma unroll
                            for (int i = 0; i < 8; ++i) ar[i][hh] = fmaf(w, (float)vh[i], ar[i][hh]);
                        }
                        __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                        dload(t + 4 * DD, kst[d], vst[d]);
                        __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        ar[i][hh] += __shfl_xor(ar[i][hh], 16);
                        ar[i][hh] += __shfl_xor(ar[i][hh], 32);
                    }
                if (tl == 0) { // lanes 0..15 own coordinates c0..c0+7 of slot 0 (still zero)
#pragma unroll
                    for (int i = 0; i < 8; ++i) lds_put<G>(acc + (c0 + i) * CS, ar[i]);
                }
                __syncthreads();
            }

            // ---- sparse rows [t0, t1)
            // Rows go in passes of D ring slots x TPI rows.  Key and value planes
            // sit in separate ring slots: a pass's scores come from the K slots, one
            // rescale test covers the whole pass, then its values are scattered from
            // the V slots.  Slots are reloaded as soon as they are consumed.
            if (t0 < t1) {
                const int tl = lane % TPI, sub = lane / TPI;
                float *my_acc = acc + tl * G; // coordinate c of this slot: my_acc[c * CS]
                const uint8_t *kidx = a.kidx, *vidx = a.vidx;
                const uint8_t *kval = a.kval, *vval = a.vval; // VB bytes per entry
                if constexpr (!PAGED) { // per-unit base in scalar registers, 32-bit lane offsets
                    const int64_t ub = ((int64_t)b * a.H + h) * a.geom.n_cap; // the unit's first row slot
                    kidx += ub * KS;
                    vidx += ub * KSV;
                    kval += ub * KS * VB;
                    vval += ub * KSV * VB;
                }
                // row slot of row r0 + tl (rows past t1 re-read the last row and
                // are masked); paged rows whose block-table entry is not a block of
                // the pool read block 0 and are dropped
                auto slice = [&](int r0, bool &ok) -> int64_t {
                    const int r = min(r0 + tl, t1 - 1);
                    if constexpr (PAGED) {
                        const int blk = a.geom.bt[(int64_t)b * a.geom.max_blocks + r / a.geom.bs];
                        ok = blk >= 0 && blk < a.geom.num_blocks;
                        const int64_t bb = ok ? blk : 0;
                        return (bb * a.H + h) * a.geom.bs + r % a.geom.bs;
                    } else {
                        ok = true;
                        return r;
                    }
                };
                KSlot<E, VB> rk[D];
                VSlot<EV, VB> rv[D];
                // Contiguous rows: a buffer resource per plane covers rows r0 .. t1-1
                // (scalar arithmetic); each lane reads its slice at a fixed offset and
                // rows past t1 read zeros (masked by valid).  Paged rows go through the
                // block table one row at a time.
                const uint32_t lane_off = (uint32_t)(tl * KS + sub * E);     // key planes
                const uint32_t lane_off_v = (uint32_t)(tl * KSV + sub * EV); // value planes
                // Paged pools whose blocks hold a power-of-two multiple of TPI rows:
                // the TPI rows of a ring slot start at a multiple of TPI (t0 is a
                // multiple of 16, passes of D x TPI rows), so they lie in one block, whose id is
                // wave-uniform and comes through the scalar cache.  The slot then
                // reads through a buffer resource on that block like the contiguous
                // layout.  The ids of a pass's slots are fetched together at the top
                // of the pass (one wait for all of them), used by the key loads and
                // kept in scalar registers for the value loads of the next pass.
                // Other block sizes look the block up per row.
                constexpr bool slot_blocks = PAGED && SLOTS;
                const int bsh = PAGED ? __builtin_ctz((unsigned)a.geom.bs) : 0; // log2 of the block size
                const int64_t tab = PAGED ? (int64_t)b * a.geom.max_blocks : 0;  // the sequence's table row
                const int64_t blk_rows = PAGED ? (int64_t)a.H * a.geom.bs : 0;   // row slots of one block
                const int64_t h_rows = PAGED ? (int64_t)h * a.geom.bs : 0;       // this head's rows in a block
                // block id of the ring slot at row r0: -1 past the piece (the table may
                // end there; the slot reads nothing), -2 an entry that is not a block of
                // the pool (the slot reads nothing and its rows are dropped)
                auto slot_block = [&](int r0) -> int {
                    if (!PAGED || !slot_blocks || r0 >= t1) return -1;
                    const int blk = a.geom.bt[tab + (r0 >> bsh)];
                    return (blk >= 0 && blk < a.geom.num_blocks) ? blk : -2;
                };
                // row slot of the ring slot at r0 in block blk and the number of its rows
                // to read (rows past t1 read zeros and are masked by row)
                auto slot_base = [&](int r0, int blk, uint32_t &rows) -> int64_t {
                    rows = blk >= 0 ? (uint32_t)min(t1 - r0, TPI) : 0u;
                    return blk >= 0 ? (int64_t)blk * blk_rows + h_rows + (r0 & (a.geom.bs - 1)) : 0;
                };
                // Ring slot d of the pass starting at row rp.  Contiguous rows: one
                // buffer resource per plane and pass, covering rows rp .. t1-1 (the
                // rest read as zeros), and slot d at a constant offset from it, so
                // the per-slot address work is an immediate offset.
                // (blk: the slot's block id from slot_block, paged pools only)
                auto load_k = [&](int rp, int d, KSlot<E, VB> &st, int blk) {
                    const int r0 = rp + d * TPI;
                    if (PAGED && !slot_blocks) {
                        const int64_t o = (int64_t)slice(r0, st.ok) * KS + sub * E;
                        load_words<E>(kidx + o, st.ki);
                        load_words<VB * E>(kval + o * VB, st.kv);
                    } else if constexpr (PAGED) {
                        uint32_t rows;
                        st.ok = blk != -2;
                        const int64_t base = slot_base(r0, blk, rows) * KS;
                        buffer_words<E>(buffer_rsrc(kidx + base, rows * KS), lane_off, st.ki);
                        buffer_words<VB * E>(buffer_rsrc(kval + base * VB, rows * KS * VB), VB * lane_off, st.kv);
                    } else {
                        const uint32_t rows = (uint32_t)max(t1 - rp, 0), off = lane_off + d * TPI * KS;
                        st.ok = true;
                        buffer_words<E>(buffer_rsrc(kidx + (int64_t)rp * KS, rows * KS), off, st.ki);
                        buffer_words<VB * E>(buffer_rsrc(kval + (int64_t)rp * KS * VB, rows * KS * VB), VB * off, st.kv);
                    }
                };
                auto load_v = [&](int rp, int d, VSlot<EV, VB> &st, int blk) {
                    const int r0 = rp + d * TPI;
                    if (PAGED && !slot_blocks) {
                        bool ok;
                        const int64_t o = (int64_t)slice(r0, ok) * KSV + sub * EV;
                        load_words<EV>(vidx + o, st.vi);
                        load_words<VB * EV>(vval + o * VB, st.vv);
                    } else if constexpr (PAGED) {
                        uint32_t rows;
                        const int64_t base = slot_base(r0, blk, rows) * KSV;
                        buffer_words<EV>(buffer_rsrc(vidx + base, rows * KSV), lane_off_v, st.vi);
                        buffer_words<VB * EV>(buffer_rsrc(vval + base * VB, rows * KSV * VB), VB * lane_off_v, st.vv);
                    } else {
                        const uint32_t rows = (uint32_t)max(t1 - rp, 0), off = lane_off_v + d * TPI * KSV;
                        buffer_words<EV>(buffer_rsrc(vidx + (int64_t)rp * KSV, rows * KSV), off, st.vi);
                        buffer_words<VB * EV>(buffer_rsrc(vval + (int64_t)rp * KSV * VB, rows * KSV * VB), VB * off,
                                              st.vv);
                    }
                };
                // value entries at row positions >= k_v are padding (index 0, value
                // +0): they add nothing, but their write-back could overwrite the
                // update of a kept entry at index 0, so they are not written (key
                // padding only adds q[0] * 0 to a score)
                const int kept = a.k_v - sub * EV;

                // Software pipeline over passes of D * TPI rows: while the values of
                // pass i are scattered, the scores of pass i + 1 are gathered, so the
                // LDS and memory waits of one overlap the arithmetic of the other.
                // Ring loads are issued in the order they are consumed (K slot d for
                // two passes ahead, then V slot d for one pass ahead).
                constexpr int P = D * TPI;
                // g = 4 with 16 slots keeps scores transposed (one head per lane):
                // m_me / ls_me are the running max and weight sum of head hme of
                // this lane's row slot
                const int hme = transposed_head(lane);
                float m_me = kNoScore, ls_me = 0.f;
                if constexpr (kT) {
                    m_me = m[0];
#pragma unroll
                    for (int hh = 1; hh < G; ++hh) m_me = hme == hh ? m[hh] : m_me;
                }
                auto reduce_scores = [&](float (&sk)[G], bool valid, float (&out)[G]) {
                    if constexpr (kT) {
                        if constexpr (TPI == 8) { // the two lanes of a slot in each 16-lane row
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) sk[hh] += dpp<0x128>(sk[hh]);
                        }
                        const float t = transposed_sum4(sk[0], sk[1], sk[2], sk[3]);
                        out[0] = valid ? t : -INFINITY;
                    } else {
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) {
                            const float gs = slot_sum<TPI>(sk[hh]); // all lanes take part in the permutes
                            out[hh] = valid ? gs : -INFINITY;
                        }
                    }
                };
                // scores of one ring slot (gather q_hat at the stored key indices);
                // rows past t1 get -inf
                auto score = [&](int r0, const KSlot<E, VB> &st, float (&sc)[G]) {
                    const bool valid = (r0 + tl < t1) && st.ok;
                    float q[E][G], s[G]; // all gathers in flight before the first product
#pragma unroll
                    for (int e = 0; e < E; ++e) lds_get<G>(qs + byte_at(st.ki, e) * G, q[e]);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float v = value_at<VB>(st.kv, e);
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) s[hh] = fmaf(q[e][hh], v, s[hh]);
                    }
                    reduce_scores(s, valid, sc);
                };
                // block ids of paged ring slots: bk for the pass whose keys were
                // loaded last (its values load next), bn for the one after
                int bk[D], bn[D];
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    bk[d] = slot_block(t0 + d * TPI);
                    bn[d] = slot_block(t0 + P + d * TPI);
                }
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    load_k(t0, d, rk[d], bk[d]);
                    __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                }
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    load_v(t0, d, rv[d], bk[d]);
                    __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                }
                float sc[D][G];
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    score(t0 + d * TPI, rk[d], sc[d]);
                    __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                    load_k(t0 + P, d, rk[d], bn[d]);
                    __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                }
#pragma unroll
                for (int d = 0; d < D; ++d) bk[d] = bn[d];

                for (int rb = t0; rb < t1; rb += P) {
#pragma unroll
                    for (int d = 0; d < D; ++d) bn[d] = slot_block(rb + 2 * P + d * TPI); // keys loaded this pass
                    // rescale test for pass rb (wave-uniform, rare)
                    float dm = -INFINITY;
#pragma unroll
                    for (int d = 0; d < D; ++d) {
                        if constexpr (kT) {
                            dm = fmaxf(dm, sc[d][0] - m_me);
                        } else {
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) dm = fmaxf(dm, sc[d][hh] - m[hh]);
                        }
                    }
                    if constexpr (kT) {
                        if (__any(dm > kRescaleSlack)) {
                            float mx = sc[0][0];
#pragma unroll
                            for (int d = 1; d < D; ++d) mx = fmaxf(mx, sc[d][0]);
                            const float mn = fmaxf(m_me, row_max16(mx)); // a row holds one head
                            const float f_me = fast_exp2(m_me - mn);
                            m_me = mn;
                            ls_me *= f_me;
                            float f[4];
                            transposed_broadcast4(f_me, f);
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) ld[hh] *= f[hh];
                            const f32x4 fv = {f[0], f[1], f[2], f[3]};
                            for (int i = lane * 4; i < NACC; i += kWave * 4) *(f32x4 *)(acc + i) *= fv;
                        }
                    } else if (__any(dm > kRescaleSlack)) {
                        float f[G];
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) {
                            float mx = sc[0][hh];
#pragma unroll
                            for (int d = 1; d < D; ++d) mx = fmaxf(mx, sc[d][hh]);
                            const float mn = fmaxf(m[hh], wave_max(mx));
                            f[hh] = fast_exp2(m[hh] - mn);
                            m[hh] = mn;
                            ls[hh] *= f[hh];
                            ld[hh] *= f[hh];
                        }
                        // a 4-float group at index i covers heads (i + j) % G; i % 8 is (lane & 1) * 4
                        f32x4 fv;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            float x = f[j % G];
                            if constexpr (G == 8) x = (lane & 1) ? f[4 + j] : f[j];
                            fv[j] = x;
                        }
                        for (int i = lane * 4; i < NACC; i += kWave * 4) *(f32x4 *)(acc + i) *= fv;
                    }
                    float sn[D][G];
#pragma unroll
                    for (int d = 0; d < D; ++d) {
                        // both LDS batches in flight before any arithmetic: the value
                        // reads of pass rb and the key gathers of pass rb + P
                        const KSlot<E, VB> &ks = rk[d];
                        const VSlot<EV, VB> &vs = rv[d];
                        float o[EV][G], q[E][G];
                        float *vaddr[EV];
#pragma unroll
                        for (int e = 0; e < EV; ++e) {
                            if constexpr (CS * 4 == 256) // 16 slots x 4 heads: one v_perm per address
                                vaddr[e] = (float *)((char *)acc + acc_offset_256(vs.vi, e, (uint32_t)(tl * G * 4)));
                            else
                                vaddr[e] = my_acc + byte_at(vs.vi, e) * CS;
                        }
#pragma unroll
                        for (int e = 0; e < EV; ++e) lds_get<G>(vaddr[e], o[e]);
#pragma unroll
                        for (int e = 0; e < E; ++e) lds_get<G>(qs + byte_at(ks.ki, e) * G, q[e]);
                        // values of pass rb
                        float w[G];
                        if constexpr (kT) {
                            const float w_me = fast_exp2(sc[d][0] - m_me);
                            ls_me += w_me;
                            transposed_broadcast4(w_me, w);
                        } else {
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) {
                                w[hh] = fast_exp2(sc[d][hh] - m[hh]);
                                ls[hh] += w[hh];
                            }
                        }
#pragma unroll
                        for (int e = 0; e < EV; ++e) {
                            const float v = value_at<VB>(vs.vv, e);
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) o[e][hh] = fmaf(w[hh], v, o[e][hh]);
                        }
#pragma unroll
                        for (int e = 0; e < EV; ++e)
                            if (!PAD || e < kept) lds_put<G>(vaddr[e], o[e]);
                        // scores of pass rb + P
                        const int r1 = rb + P + d * TPI;
                        const bool valid = (r1 + tl < t1) && ks.ok;
                        float sk[G];
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) sk[hh] = 0.f;
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const float v = value_at<VB>(ks.kv, e);
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) sk[hh] = fmaf(q[e][hh], v, sk[hh]);
                        }
                        reduce_scores(sk, valid, sn[d]);
                        __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                        load_k(rb + 2 * P, d, rk[d], bn[d]);
                        __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                        load_v(rb + P, d, rv[d], bk[d]);
                        __builtin_amdgcn_sched_barrier(kKeepLoadOrder);
                    }
#pragma unroll
                    for (int d = 0; d < D; ++d) {
                        bk[d] = bn[d];
#pragma unroll
                        for (int hh = 0; hh < G; ++hh) sc[d][hh] = sn[d][hh];
                    }
                }
                if constexpr (kT) {
                    // back to per-head registers: a row holds one head; its 16 lanes
                    // hold the weight sums of the row slots (16 slots once each, or 8
                    // slots twice each: halved, exactly)
                    float mh[4], lh[4];
                    transposed_broadcast4(m_me, mh);
                    transposed_broadcast4(group_sum<16>(ls_me) * (TPI == 8 ? 0.5f : 1.0f), lh);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        m[hh] = mh[hh];
                        ls[hh] = lh[hh]; // the head's whole sum, in every lane
                    }
                }
            }
            __syncthreads();

            // ---- partials of the piece: (m, l) and the sum of the accumulator copies
            const int64_t pbase = piece * G; // + hh per head
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                // generic path: every lane of a row slot added the slot's weights, so
                // the wave sum counts each LPT times (exactly: LPT is a power of two)
                const float lsum = kT ? ls[hh] : wave_sum(ls[hh]) * (1.0f / LPT);
                const float lt = lsum + wave_sum(ld[hh]);
                if (lane == 0) {
                    a.part_ml[(pbase + hh) * 2] = m[hh];
                    a.part_ml[(pbase + hh) * 2 + 1] = lt;
                }
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // lane walks the slots of its coordinate starting at slot lane % TPI,
                // so the 16 lanes of an LDS phase read 16 different bank quads
                const int c = lane + half * kWave;
                float o[G], t[G];
                lds_get<G>(acc + c * CS + (lane % TPI) * G, o);
#pragma unroll
                for (int cp = 1; cp < TPI; ++cp) {
                    lds_get<G>(acc + c * CS + ((lane + cp) % TPI) * G, t);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) o[hh] += t[hh];
                }
#pragma unroll
                for (int hh = 0; hh < G; ++hh) a.part_o[(pbase + hh) * kD + c] = o[hh];
            }
            __syncthreads(); // the next piece rewrites the queries and accumulators
        }
        P += uw.len * a.H;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int G, int KS, int KSV, bool PAGED, int VB, bool SLOTS>
inline void launch_split_v(const SplitArgs &a, hipStream_t s)
{
    const dim3 grid(a.W), block(kWave);
    if (a.k_v < KSV)
        hipLaunchKernelGGL((k_split<G, KS, KSV, PAGED, true, VB, SLOTS>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_split<G, KS, KSV, PAGED, false, VB, SLOTS>), grid, block, 0, s, a);
}

template <int G, int KS, int KSV, bool PAGED, bool SLOTS>
inline void launch_split_k(const SplitArgs &a, hipStream_t s)
{
    if (a.geom.vbytes == 1)
        launch_split_v<G, KS, KSV, PAGED, 1, SLOTS>(a, s);
    else
        launch_split_v<G, KS, KSV, PAGED, 2, SLOTS>(a, s);
}

// key row width x value row width: equal, or one twice the other
template <int G, bool PAGED, bool SLOTS = false>
inline hipError_t launch_split_g(const SplitArgs &a, hipStream_t s)
{
    const int ks = a.geom.ks, ksv = a.geom.ks_v;
    switch (ks * 1000 + ksv) {
    case 8008: launch_split_k<G, 8, 8, PAGED, SLOTS>(a, s); break;
    case 8016: launch_split_k<G, 8, 16, PAGED, SLOTS>(a, s); break;
    case 16008: launch_split_k<G, 16, 8, PAGED, SLOTS>(a, s); break;
    case 16016: launch_split_k<G, 16, 16, PAGED, SLOTS>(a, s); break;
    case 16032: launch_split_k<G, 16, 32, PAGED, SLOTS>(a, s); break;
    case 32016: launch_split_k<G, 32, 16, PAGED, SLOTS>(a, s); break;
    case 32032: launch_split_k<G, 32, 32, PAGED, SLOTS>(a, s); break;
    case 32064: launch_split_k<G, 32, 64, PAGED, SLOTS>(a, s); break;
    case 64032: launch_split_k<G, 64, 32, PAGED, SLOTS>(a, s); break;
    case 64064: launch_split_k<G, 64, 64, PAGED, SLOTS>(a, s); break;
    case 64128: launch_split_k<G, 64, 128, PAGED, SLOTS>(a, s); break;
    case 128064: launch_split_k<G, 128, 64, PAGED, SLOTS>(a, s); break;
    case 128128: launch_split_k<G, 128, 128, PAGED, SLOTS>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace swan
