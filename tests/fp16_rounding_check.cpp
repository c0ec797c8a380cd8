// Host check of swan::d2h_odd (csrc/fp16_round.h) against the compiler
// runtime's direct double -> fp16 conversion (round to nearest even): every
// finite fp16 value and every midpoint between neighbours, each with the
// doubles up to 3 ulps either side and a float ulp either side, both signs;
// 20 million random doubles over 2^-30 .. 2^18; 5 million points scattered
// around random midpoints; zeros, infinities, the overflow boundary.
// Prints "<checked> checked, <mismatches> mismatches"; exit status 1 on any.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

#include "fp16_round.h"

static uint64_t bad = 0, n = 0;

static void check(double x)
{
    ++n;
    const uint16_t want = __builtin_bit_cast(uint16_t, (_Float16)x);
    const uint16_t got = swan::d2h_odd(x);
    if (want != got) {
        if (bad < 10) std::printf("mismatch x=%.17g: runtime %04x d2h_odd %04x\n", x, want, got);
        ++bad;
    }
}

static double half_value(uint16_t h) { return (double)(float)__builtin_bit_cast(_Float16, h); }

int main()
{
    std::mt19937_64 g(1);
    for (uint32_t h = 0; h < 0x7c00; ++h) {
        const double v = half_value((uint16_t)h), nx = half_value((uint16_t)(h + 1));
        const double mid = (v + nx) / 2; // exact in double
        for (double base : {v, mid}) {
            for (int s = -3; s <= 3; ++s) {
                double y = base;
                for (int i = 0; i < s; ++i) y = std::nextafter(y, (double)INFINITY);
                for (int i = 0; i < -s; ++i) y = std::nextafter(y, -(double)INFINITY);
                check(y);
                check(-y);
            }
            const double fu = std::ldexp(std::fabs(base) + 1e-300, -24);
            check(base + fu);
            check(base - fu);
        }
    }
    std::uniform_real_distribution<double> e(-30, 18), u(1, 2);
    for (int i = 0; i < 20000000; ++i) {
        double x = std::ldexp(u(g), (int)std::floor(e(g)));
        check((g() & 1) ? -x : x);
    }
    for (int i = 0; i < 5000000; ++i) {
        const uint16_t h = (uint16_t)(g() % 0x7bff);
        const double v = half_value(h), nx = half_value((uint16_t)(h + 1)), mid = (v + nx) / 2;
        const double d = (nx - v) * std::ldexp((double)(int64_t)(g() % 2000001) - 1000000, -40);
        check(mid + d);
        check(-(mid + d));
    }
    for (double x : {0.0, -0.0, 65504.0, 65519.99, 65520.0, 65520.0000001, 65536.0, 1e10, 1e300, 5.96e-8, 2.98e-8,
                     2.9802322387695312e-08, 1e-300, -1e-300, (double)INFINITY, -(double)INFINITY})
        check(x);
    std::printf("%llu checked, %llu mismatches\n", (unsigned long long)n, (unsigned long long)bad);
    return bad != 0;
}
