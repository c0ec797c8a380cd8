// topk_rows.h -- the magnitude top-k of wave_prune_row (swan_internal.h),
// split in two so that a wave pruning many rows can interleave them: the
// same ranking (fp16 magnitude bits descending, index ascending), the same
// row layout, bit for bit (SWAN page, pruning paragraph: each evicted
// vector keeps its k largest-magnitude coordinates).
//
// wave_topk_threshold finds, for each of NR rows at once, the k-th largest
// magnitude T bit by bit from the top: the largest T with at least k
// magnitudes >= T (ballots and popcounts only).  The NR searches are
// independent; every ballot of a bit step is taken before any popcount, so
// the compares write separate scalar pairs and their chains overlap.
// wave_write_topk then writes one row given its T.  Both must be called by
// all 64 lanes; a row's coordinate lane sits in `lo`, lane + 64 in `hi`.
#pragma once

#include "swan_internal.h"

namespace swan {

template <int NR>
__device__ __forceinline__ void wave_topk_threshold(const uint16_t (&lo)[NR], const uint16_t (&hi)[NR],
                                                    const int (&k)[NR], uint32_t (&T)[NR])
{
    uint32_t mlo[NR], mhi[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        mlo[n] = lo[n] & 0x7fffu;
        mhi[n] = hi[n] & 0x7fffu;
        T[n] = 0;
    }
#pragma unroll
    for (int bit = 14; bit >= 0; --bit) {
        uint64_t blo[NR], bhi[NR];
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const uint32_t c = T[n] | (1u << bit);
            blo[n] = __ballot(mlo[n] >= c);
            bhi[n] = __ballot(mhi[n] >= c);
        }
#pragma unroll
        for (int n = 0; n < NR; ++n)
            if (__popcll(blo[n]) + __popcll(bhi[n]) >= k[n]) T[n] |= 1u << bit;
    }
}

// The k kept coordinates of a row with threshold T, ascending by index, and
// ks - k zero padding entries; values copied (vbytes 2) or rounded to E4M3.
__device__ __forceinline__ void wave_write_topk(int lane, uint16_t lo, uint16_t hi, uint32_t T, int k, int ks,
                                                uint8_t *idx_row, uint8_t *val_row, int vbytes)
{
    auto put = [&](int o, uint16_t v) {
        if (vbytes == 1)
            val_row[o] = h2e4m3(v);
        else
            ((uint16_t *)val_row)[o] = v;
    };
    const uint32_t mlo = lo & 0x7fffu, mhi = hi & 0x7fffu;
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

} // namespace swan
