// rope_trig.h -- sine and cosine of a RoPE angle in double, for the prefill
// conversion's per-coordinate rotation (every coordinate pair of every token
// has its own angle t theta_i, so the rotation's cost is that of sincos).
//
// Cody-Waite argument reduction: k = nearest integer to x 2/pi, and
// r = x - k pi/2 with pi/2 split as P1 + P2 + P3 (33, 33 and 53 significant
// bits, the exact leading bits of pi/2), so that k P1 and k P2 are exact for
// k < 2^20 and x - k P1 is exact (Sterbenz); r is then within one ulp of its
// true value.  sin r and cos r come from their Taylor series to r^19 and
// r^18 (on |r| <= pi/4 the next terms are below 1e-21), in Horner form; the
// quadrant k mod 4 swaps and negates them.  Measured against long double
// over every angle t theta_i of 131072 positions and 64 frequencies for two
// bases, and 4 million uniform arguments below 2^18: absolute error at most
// 1.6e-16 (tests/test_device_math_cpu.py).  Arguments of 2^20 pi/2 and more
// (positions past ~1.6 million at the fastest frequency) take the library's
// sincos instead.
#pragma once

namespace swan {

__host__ __device__ inline void rope_sincos(double x, double &sn, double &cs)
{
    constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
    constexpr double kP1 = 0x1.921fb54400000p+0, kP2 = 0x1.0b4611a600000p-34, kP3 = 0x1.3198a2e037073p-69;
    constexpr double kLimit = 0x1.921fb54400000p+20; // 2^20 P1
    if (!(x < kLimit)) {
        sincos(x, &sn, &cs);
        return;
    }
    const double k = __builtin_rint(x * kTwoOverPi);
    double r = __builtin_fma(-k, kP1, x);
    r = __builtin_fma(-k, kP2, r);
    r = __builtin_fma(-k, kP3, r);
    const double z = r * r;
    double p = -1.0 / 121645100408832000.0; // -1/19!
    p = __builtin_fma(p, z, 1.0 / 355687428096000.0);
    p = __builtin_fma(p, z, -1.0 / 1307674368000.0);
    p = __builtin_fma(p, z, 1.0 / 6227020800.0);
    p = __builtin_fma(p, z, -1.0 / 39916800.0);
    p = __builtin_fma(p, z, 1.0 / 362880.0);
    p = __builtin_fma(p, z, -1.0 / 5040.0);
    p = __builtin_fma(p, z, 1.0 / 120.0);
    p = __builtin_fma(p, z, -1.0 / 6.0);
    const double s = __builtin_fma(r * z, p, r);
    double c = -1.0 / 6402373705728000.0; // -1/18!
    c = __builtin_fma(c, z, 1.0 / 20922789888000.0);
    c = __builtin_fma(c, z, -1.0 / 87178291200.0);
    c = __builtin_fma(c, z, 1.0 / 479001600.0);
    c = __builtin_fma(c, z, -1.0 / 3628800.0);
    c = __builtin_fma(c, z, 1.0 / 40320.0);
    c = __builtin_fma(c, z, -1.0 / 720.0);
    c = __builtin_fma(c, z, 1.0 / 24.0);
    c = __builtin_fma(c, z, -0.5);
    c = __builtin_fma(z, c, 1.0);
    // quadrant k mod 4: (sin, cos) = (s, c), (c, -s), (-s, -c), (-c, s)
    const int n = (int)k & 3;
    const double a = (n & 1) ? c : s, b = (n & 1) ? s : c;
    sn = (n & 2) ? -a : a;
    cs = ((n + 1) & 2) ? -b : b;
}

} // namespace swan
