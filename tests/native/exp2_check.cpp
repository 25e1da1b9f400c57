// Host build of the library's fp64 exp2 helpers, checked against libm's exp2l: the
// series exp2_f64, and the table method of the fp32 streaming pass (2^(a/L) from a
// table of 2^(j/L) and a short series).
// Prints: max_ulp mean_rel n exp2(-inf) exp2(nan) exp2(0) table_max_rel table_n
#include <cmath>
#include <cstdio>
#include <cstdint>
#include "sv_stream.h"

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

    // the table method over the arguments the streaming pass gives it: a in
    // [-1000 L, L / 2] (exponents from the clamp at 2^-1000 up to rounding above 0)
    static double tab[sv::kTabLen];
    for (int j = 0; j < sv::kTabLen; ++j) tab[j] = sv::exp2_tab_entry(j);
    const sv::Exp2Tab t{tab, 0};
    const double L = (double)sv::kTabLen;
    double tab_max_rel = 0.0;
    long tn = 0;
    for (long i = 0; i < 2000000; ++i) {
        state = state * 6364136223846793005ull + 1442695040888963407ull;
        const double a = -1000.0 * L + 1000.5 * L * (double)(state >> 11) / 9007199254740992.0;
        const double got = sv::exp2_tab_add(sv::exp2_tab_read(a, t), 0.0);
        const long double ref = exp2l((long double)a / (long double)L);
        const double rel = (double)fabsl(((long double)got - ref) / ref);
        if (rel > tab_max_rel) tab_max_rel = rel;
        ++tn;
    }
    std::printf("%.4f %.3e %ld %g %g %g %.3e %ld\n", max_ulp, sum_rel / n, n, special[0], special[1], special[2],
                tab_max_rel, tn);
    return 0;
}
