// fp16_round.h -- fp16 bits of a double, rounded once to nearest even,
// without branches: the double is rounded to float with rounding to odd
// (round toward zero, then set the last bit when the result is inexact),
// and that float to fp16 with the hardware's round-to-nearest-even.
// Rounding to odd at a precision at least two bits wider than the target
// makes the second rounding correct (S. Boldo, G. Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE Transactions on Computers 57(4), 2008); float carries 24 significand
// bits against fp16's 11, and fp16's subnormal range lies inside float's
// normal range.  Same result as d2h (swan_internal.h) for every double.
#pragma once

#include <stdint.h>

namespace swan {

__host__ __device__ inline uint16_t d2h_odd(double x)
{
    const float f = (float)x; // nearest float
    const double back = (double)f;
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    b -= (__builtin_fabs(back) > __builtin_fabs(x)) ? 1u : 0u; // the neighbour toward zero
    b |= (back != x) ? 1u : 0u;                                   // odd when inexact
    return __builtin_bit_cast(uint16_t, (_Float16)__builtin_bit_cast(float, b));
}

} // namespace swan
