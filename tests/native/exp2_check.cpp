// Host build of the library's fp64 exp2 helper, checked against libm's exp2l.
// Prints: max_ulp mean_rel n
#include <cmath>
#include <cstdio>
#include <cstdint>
#include "sv_internal.h"

int main()
{
    double max_ulp = 0.0, sum_rel = 0.0;
    long n = 0;
    uint64_t state = 0x9e3779b97f4a7c15ull;
    for (long i = 0; i < 4000000; ++i) {
        state = state * 6364136223846793005ull + 1442695040888963407ull;
        const double x = -1070.0 + 2093.0 * (double)(state >> 11) / 9007199254740992.0;
        const double got = sv::exp2_f64(x);
        const long double ref = exp2l((long double)x);
        if (ref < 2.3e-308L) continue;   // subnormal results are not used
        const double ulp = std::ldexp(1.0, std::ilogb((double)ref) - 52);
        const double e = (double)(((long double)got - ref) / ulp);
        if (std::fabs(e) > max_ulp) max_ulp = std::fabs(e);
        sum_rel += (double)(((long double)got - ref) / ref);
        ++n;
    }
    const double special[3] = {sv::exp2_f64(-INFINITY), sv::exp2_f64(NAN), sv::exp2_f64(0.0)};
    std::printf("%.4f %.3e %ld %g %g %g\n", max_ulp, sum_rel / n, n, special[0], special[1], special[2]);
    return 0;
}
