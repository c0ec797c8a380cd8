// Host check of swan::rope_sincos (csrc/rope_trig.h) against long double
// sinl / cosl: every angle t theta_i (t < 131072, theta_i = base^(-i/64),
// i < 64) for bases 10000 and 500000, 4 million uniform arguments below
// 2^18, and arguments around the switch to the library routine.  Prints the
// largest absolute error; exit status 1 if it exceeds 2.3e-16.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

#include "rope_trig.h"

int main()
{
    double worst = 0, worst_x = 0;
    uint64_t n = 0;
    auto check = [&](double x) {
        double s, c;
        swan::rope_sincos(x, s, c);
        const long double S = sinl((long double)x), C = cosl((long double)x);
        const double e = (double)fmaxl(fabsl((long double)s - S), fabsl((long double)c - C));
        if (e > worst) {
            worst = e;
            worst_x = x;
        }
        ++n;
    };
    for (double base : {10000.0, 500000.0})
        for (int i = 0; i < 64; ++i) {
            const double theta = std::pow(base, -(double)i / 64.0);
            for (int t = 0; t < 131072; ++t) check((double)t * theta);
        }
    std::mt19937_64 g(3);
    std::uniform_real_distribution<double> u(0, 262144.0);
    for (int i = 0; i < 4000000; ++i) check(u(g));
    const double lim = 0x1.921fb54400000p+20;
    for (int d = -1000; d <= 1000; ++d) check(lim + d * 0.37);
    std::printf("%llu arguments, largest absolute error %.3g at x = %.17g\n", (unsigned long long)n, worst, worst_x);
    return worst > 2.3e-16;
}
