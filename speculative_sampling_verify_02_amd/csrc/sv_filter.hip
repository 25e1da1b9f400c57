// Top-k and top-p filtering of p and q before the test.
//
// The pages require every such filter to be applied to both the target and the
// drafter distribution before the accept test (rayaq.ca "Speculative decoding",
// section "Why the output is exactly the target's", last paragraph, and section
// "Tradeoffs").  Each filter keeps the tokens whose logit is at least a per-vector
// threshold theta:
//   top-k: theta_k is the k-th largest logit, counted with multiplicity (tokens tied
//          with it are kept);
//   top-p: on the distribution left by top-k, whole groups of equal logits are taken
//          in decreasing order until their probability reaches top_p; theta_p is the
//          logit of the last group taken;
//   theta = max(theta_k, theta_p).
//
// Both thresholds come from a radix select over keys that sort like the logits: the
// largest key t whose metric over {key >= t} reaches a target, where the metric is
// the count of logits (theta_k, target k) or their fp64 probability mass 2^((z - m) c)
// at the exact scale c = log2(e)/T (theta_p, target top_p times the mass left by
// top-k).  Each level histograms one 8-bit digit of the keys that share the digits
// chosen so far (LDS atomics) and one wave picks the digit where the running total
// from the top reaches the target: two levels for bf16 logits (16-bit keys), four
// for fp32.  Since the metric over {key >= t} only changes at keys of logits, the
// key found is a logit's.
//
// With top-k, a lower bound L of theta_k comes from maxima that are different logits
// of the vector (k of them reaching L hold k logits >= L); the logits >= L, at least
// k of them and usually a few times k, are gathered in LDS and every later select
// runs there, in one wave when they are at most 256 (the same selects a key bit at a
// time, with ballots).  Otherwise the selects run over the whole vector.
//
// filter_units_kernel takes those maxima from the streaming pass, which in filtered
// calls stores the maximum of every 64 consecutive logits, and reads again only the
// units that can hold the top-k; filter_kernel (vocabularies beyond its budget) takes
// them from the threads' own maxima, reading the vector from memory in every pass.
// Both replace the record of each vector that filters.
#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

constexpr int kFilterBlock = 1024;
constexpr int kFilterWaves = kFilterBlock / 64;
constexpr int kBins = 256;       // one 8-bit digit
constexpr int kMaxCand = 4096;   // logits kept in LDS by the top-k candidate path

// The thread index as a value the compiler must take as new at every call: what the
// helpers derive from it (lane, wave, LDS offsets) is recomputed where used rather
// than kept in registers.
__device__ __forceinline__ int tid_now()
{
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// 2^x in fp64 (exp2_f64) with the series' coefficients read from constant memory
// (scalar registers rather than vector registers).
static __constant__ double kExp2Table[14] = {kExp2Coef[0], kExp2Coef[1], kExp2Coef[2],  kExp2Coef[3],  kExp2Coef[4],
                                             kExp2Coef[5], kExp2Coef[6], kExp2Coef[7],  kExp2Coef[8],  kExp2Coef[9],
                                             kExp2Coef[10], kExp2Coef[11], kExp2Coef[12], kExp2Coef[13]};
__device__ __forceinline__ double fexp2(double x)
{
    return exp2_f64_by(x, [](int j) { return kExp2Table[j]; });
}

// A finite or infinite float as an unsigned key that sorts like the float.
__device__ __forceinline__ uint32_t fkey(float x)
{
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The float of key t whose bits below LOW are those of a logit of the data (bf16
// logits, LOW = 16: the low 16 bits of the float are zero).
template <int LOW>
__device__ __forceinline__ float key_val(uint32_t t)
{
    if constexpr (LOW > 0)
        if (!(t & 0x80000000u)) t |= (1u << LOW) - 1u;   // negative values: low key bits set
    return __uint_as_float((t & 0x80000000u) ? (t & 0x7fffffffu) : ~t);
}

struct FilterLds {
    static constexpr uint32_t kCap = kMaxCand;
    float cand[kMaxCand];   // logits at or above a lower bound of theta_k
    uint32_t ncand;
    uint32_t cnt[kBins];
    double mass[kBins];
    double rd[kFilterWaves];
    float rf[kFilterWaves];
    uint32_t ru[kFilterWaves];
    uint32_t rsel;          // radix select: key prefix so far
    double rabove;          // and the metric above it
    float wtheta;           // one-wave select results
    double wS;
};

// Block-wide helpers for a workgroup of NT threads; Lds is the kernel's LDS layout
// (FilterLds, or the smaller one of filter_units_kernel).
template <int NT = kFilterBlock, class Lds>
__device__ __forceinline__ double fblock_sum(double v, Lds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) sh.rd[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += sh.rd[w];
    return t;
}

// Block-wide maximum of the threads' values, NaN if any is NaN.
template <int NT = kFilterBlock, class Lds>
__device__ __forceinline__ float block_nmax(float v, Lds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    v = wave_umax_f32(v);
    if (lane == 0) sh.rf[wave] = v;
    __syncthreads();
    float m = -INFINITY;
    for (int w = 0; w < NT / 64; ++w) m = nmax(m, sh.rf[w]);
    __syncthreads();
    return m;
}

// Every logit of the vector through f(z), 8 per thread per step.  Rows that are not
// 16-byte aligned are read a 512-logit tile per wave with aligned loads shifted into
// place (load_tile_unit), the logits past V as -inf (arr, arr_bytes: the array the
// row lies in).
// Four loads per thread are issued before the first is reduced.
template <int DT, bool AL, int NT = kFilterBlock, class F>
__device__ __forceinline__ void each_logit(const void *base, int64_t V, int64_t nunits, const void *arr,
                                           uint64_t arr_bytes, F &&f)
{
    constexpr int U = 4;
    if constexpr (AL) {
        for (int64_t u0 = tid_now(); u0 < nunits; u0 += U * NT) {
            RawUnit<DT> r[U];
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (u0 + (int64_t)i * NT < nunits) r[i] = load_raw<DT, AL>(base, u0 + (int64_t)i * NT, V);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                if (u0 + (int64_t)i * NT >= nunits) break;
                float z[kUnitElems];
                unpack<DT>(r[i], z);
#pragma unroll
                for (int e = 0; e < kUnitElems; ++e) f(z[e]);
            }
        }
    } else {
        const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
        constexpr int64_t step = NT / 64;
        for (int64_t t0 = wave; t0 * kTileUnits < nunits; t0 += U * step) {
            RawUnit<DT> r[U];
#pragma unroll
            for (int i = 0; i < U; ++i)
                if ((t0 + i * step) * kTileUnits < nunits)
                    r[i] = load_tile_unit<DT>(base, t0 + i * step, V, arr, arr_bytes, lane);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                if ((t0 + i * step) * kTileUnits >= nunits) break;
                float z[kUnitElems];
                unpack<DT>(r[i], z);
#pragma unroll
                for (int e = 0; e < kUnitElems; ++e) f(z[e]);
            }
        }
    }
}

// The largest key t (bits >= LOW) whose metric over {key >= t} reaches target > 0:
// the count of the logits `each` passes (MASS false), or the sum of their weights
// 2^((z - m) c64) (MASS true).  The total metric must reach the target.
template <bool MASS, int LOW, class Src, class Lds>
__device__ __forceinline__ uint32_t radix_select(Src &&each, double target, float m, double c64, Lds &sh)
{
    const int tid = tid_now(), lane = tid & 63;
    uint32_t prefix = 0u;
    double above = 0.0;
#pragma unroll
    for (int shift = 24; shift >= LOW; shift -= 8) {
        for (int i = tid; i < kBins; i += blockDim.x) {
            if constexpr (MASS) sh.mass[i] = 0.0;
            else sh.cnt[i] = 0u;
        }
        __syncthreads();
        // keys whose digits above this one are the prefix's
        const uint32_t hi_mask = shift == 24 ? 0u : ~((1u << (shift + 8)) - 1u);
        each([&](float z) __attribute__((always_inline)) {
            const uint32_t key = fkey(z);
            if ((key & hi_mask) == prefix) {
                const int d = (int)((key >> shift) & 255u);
                if constexpr (MASS) atomicAdd(&sh.mass[d], fexp2(((double)z - (double)m) * c64));
                else atomicAdd(&sh.cnt[d], 1u);
            }
        });
        __syncthreads();
        if (tid < 64) {
            // lane l holds digits 255 - 4l down to 252 - 4l; the highest digit where
            // the running total from the top reaches the target
            double v[4], lsum = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = kBins - 1 - (lane * 4 + q);
                v[q] = MASS ? sh.mass[d] : (double)sh.cnt[d];
                lsum += v[q];
            }
            const double incl = wave_inclusive_sum(lsum, lane);
            double run = above + incl - lsum;
            int hit = -1;
            double hit_above = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (hit < 0 && run + v[q] >= target) {
                    hit = kBins - 1 - (lane * 4 + q);
                    hit_above = run;
                }
                run += v[q];
            }
            const unsigned long long hb = __ballot(hit >= 0);
            // (the total reaches the target, so some lane hits; digit 0 otherwise)
            const int l = hb ? __ffsll((long long)hb) - 1 : 0;
            const int d = hb ? __shfl(hit, l) : 0;
            const double a = hb ? __shfl(hit_above, l) : above;
            if (lane == 0) {
                sh.rsel = prefix | ((uint32_t)d << shift);
                sh.rabove = a;
            }
        }
        __syncthreads();
        prefix = sh.rsel;
        above = sh.rabove;
    }
    return prefix;
}

// ---------------------------------------------------------------------------
// One-wave selects over N keys per lane (key 0: no value), a key bit at a time with
// ballots: the same results as radix_select, without barriers or atomics.
// ---------------------------------------------------------------------------
// The largest t (bits >= LOW) with at least k keys >= t.
template <int LOW, int N>
__device__ __forceinline__ uint32_t wave_select_count(const uint32_t (&key)[N], int64_t k)
{
    uint32_t t = 0u;
    for (int b = 31; b >= LOW; --b) {
        const uint32_t c = t | (1u << b);
        int n = 0;
#pragma unroll
        for (int s = 0; s < N; ++s) n += __popcll(__ballot(key[s] >= c));
        if (n >= k) t = c;
    }
    return t;
}

// The largest t (bits >= LOW) whose keys >= t carry a total weight >= target.
template <int LOW, int N>
__device__ __forceinline__ uint32_t wave_select_mass(const uint32_t (&key)[N], const double (&w)[N], double target)
{
    uint32_t t = 0u;
    for (int b = 31; b >= LOW; --b) {
        const uint32_t c = t | (1u << b);
        double m = 0.0;
#pragma unroll
        for (int s = 0; s < N; ++s) m += key[s] >= c ? w[s] : 0.0;
        if (wave_usum_f64(m) >= target) t = c;
    }
    return t;
}

constexpr int kWaveCand = 4;   // candidates per lane of the one-wave path (256 in all)


// theta and the kept sum from at most 256 candidates in LDS, in one wave (the other
// waves wait at the barrier).
template <int LOW, class Lds>
__device__ __forceinline__ void one_wave_thresholds(uint32_t ncand, float mx, int64_t k, float tp, bool use_p,
                                                    double c64, Lds &sh, float &theta_out, double &S_out)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    if (wave == 0) {
        uint32_t key[kWaveCand];
        float z[kWaveCand];
#pragma unroll
        for (int s = 0; s < kWaveCand; ++s) {
            const uint32_t i = (uint32_t)(s * 64 + lane);
            z[s] = i < ncand ? sh.cand[i] : -INFINITY;
            key[s] = i < ncand ? fkey(z[s]) : 0u;
        }
        const uint32_t tk = wave_select_count<LOW, kWaveCand>(key, k);
        double w[kWaveCand], ws = 0.0;
#pragma unroll
        for (int s = 0; s < kWaveCand; ++s) {
            w[s] = key[s] >= tk ? fexp2(((double)z[s] - (double)mx) * c64) : 0.0;
            ws += w[s];
        }
        const double Sk = wave_usum_f64(ws);
        uint32_t tt = tk;
        double St = Sk;
        if (use_p) {
            const uint32_t tpk = wave_select_mass<LOW, kWaveCand>(key, w, (double)tp * Sk);
            if (tpk > tk) {
                tt = tpk;
                ws = 0.0;
#pragma unroll
                for (int s = 0; s < kWaveCand; ++s) ws += key[s] >= tt ? w[s] : 0.0;
                St = wave_usum_f64(ws);
            }
        }
        if (lane == 0) {
            sh.wtheta = key_val<LOW>(tt);
            sh.wS = St;
        }
    }
    __syncthreads();
    theta_out = sh.wtheta;
    S_out = sh.wS;
}

constexpr uint32_t kNoCand = 0xffffffffu;

// Thresholds of one vector whose logits are finite or -inf, with maximum mx > -inf,
// in two steps.  gather_candidates: with top-k, the logits of a superset of the
// kept ones into LDS (`gather_ge(L, f)` passes every logit >= L to f, spread over the
// threads; tmx is this thread's maximum under it); it returns their number, or
// kNoCand when the top-k bound does not apply.
template <int LOW, class GatherGe>
__device__ __forceinline__ uint32_t gather_candidates(GatherGe &&gather_ge, float tmx, float mx, int64_t k,
                                                      bool use_k, double c64, FilterLds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    // threads whose maximum is finite (each such maximum is a different logit)
    const int nmax_fin = __syncthreads_count(tmx > -INFINITY);
    if (!(use_k && k <= nmax_fin)) return kNoCand;
    // top-k candidates, above a lower bound L of theta_k: every wave with at least
    // m = ceil(k / 16) finite thread maxima takes its m-th largest, and L is the
    // least of them; n such waves hold at least n m logits >= L, so L bounds theta_k
    // from below when n m >= k (else L is the k-th largest of all thread maxima, by
    // a block-wide select)
    const int64_t m = (k + kFilterWaves - 1) / kFilterWaves;
    if (tid == 0) sh.ncand = 0u;
    {
        const uint32_t key[1] = {tmx > -INFINITY ? fkey(tmx) : 0u};
        float Lw = INFINITY;
        if (__popcll(__ballot(key[0] != 0u)) >= m) Lw = key_val<LOW>(wave_select_count<LOW, 1>(key, m));
        if (lane == 0) sh.rf[wave] = Lw;
    }
    __syncthreads();
    float L = INFINITY;
    int nw = 0;
    for (int w = 0; w < kFilterWaves; ++w) {
        const float lw = sh.rf[w];
        if (lw < INFINITY) {
            L = fminf(L, lw);
            ++nw;
        }
    }
    if ((int64_t)nw * m < k) {
        auto from_tmax = [&](auto &&f) __attribute__((always_inline)) { f(tmx); };
        L = key_val<LOW>(radix_select<false, LOW>(from_tmax, (double)k, mx, c64, sh));
    }
    // (every thread calls gather_ge: a source may need the whole wave for its loads)
    gather_ge(L, [&](float z) __attribute__((always_inline)) {
        const uint32_t i = atomicAdd(&sh.ncand, 1u);
        if (i < (uint32_t)kMaxCand) sh.cand[i] = z;
    });
    __syncthreads();
    return sh.ncand;
}

// finish_thresholds: theta = max(theta_k, theta_p) and the fp64 sum over the kept
// logits of 2^((z - mx) c64), from the candidates when they fit in LDS, else from the
// whole vector (`each(f)` passes every logit to f, spread over the threads;
// `part_sum(lower)` is this thread's share of the sum over the logits >= lower).
// The thresholds and the kept sum from ncand <= Lds::kCap top-k candidates in LDS:
// in one wave up to 256 of them, else by block-wide radix selects.
template <int LOW, int NT = kFilterBlock, class Lds>
__device__ __forceinline__ void cand_thresholds(uint32_t ncand, float mx, int64_t k, float tp, bool use_p,
                                                double c64, Lds &sh, float &theta_out, double &S_out)
{
    const int tid = tid_now();
    if (ncand <= (uint32_t)(kWaveCand * 64)) {
        one_wave_thresholds<LOW>(ncand, mx, k, tp, use_p, c64, sh, theta_out, S_out);
        return;
    }
    {
        {
            auto from_cand = [&](auto &&f) __attribute__((always_inline)) {
                for (uint32_t i = tid; i < ncand; i += NT) f(sh.cand[i]);
            };
            float theta = key_val<LOW>(radix_select<false, LOW>(from_cand, (double)k, mx, c64, sh));
            auto cand_sum = [&](float lower) {
                double s = 0.0;
                from_cand([&](float z) {
                    if (z >= lower) s += fexp2(((double)z - (double)mx) * c64);
                });
                return fblock_sum<NT>(s, sh);
            };
            double S = cand_sum(theta);
            if (use_p) {
                const float lk = theta;
                auto kept = [&](auto &&f) __attribute__((always_inline)) {
                    from_cand([&](float z) __attribute__((always_inline)) {
                        if (z >= lk) f(z);
                    });
                };
                const float tp_val = key_val<LOW>(radix_select<true, LOW>(kept, (double)tp * S, mx, c64, sh));
                if (tp_val > theta) {
                    theta = tp_val;
                    S = cand_sum(theta);
                }
            }
            theta_out = theta;
            S_out = S;
        }
    }
}

template <int LOW, int NT = kFilterBlock, class Each, class PartSum, class Lds>
__device__ __forceinline__ void finish_thresholds(Each &&each, PartSum &&part_sum, uint32_t ncand, float mx,
                                                  int64_t k, float tp, bool use_k, bool use_p, double c64,
                                                  Lds &sh, float &theta_out, double &S_out)
{
    if (ncand != kNoCand && ncand <= Lds::kCap) {
        cand_thresholds<LOW, NT>(ncand, mx, k, tp, use_p, c64, sh, theta_out, S_out);
        return;
    }
    // selects over the whole vector; theta_k needs at least k finite logits
    uint32_t nfin = 0u;
    each([&](float z) {
        if (z > -INFINITY) ++nfin;
    });
    nfin = (uint32_t)fblock_sum<NT>((double)nfin, sh);
    float theta = -INFINITY;
    if (use_k && (uint64_t)k <= nfin) theta = key_val<LOW>(radix_select<false, LOW>(each, (double)k, mx, c64, sh));
    double S = fblock_sum<NT>(part_sum(theta), sh);
    if (use_p) {
        const float lk = theta;
        auto kept = [&](auto &&f) {
            each([&](float z) {
                if (z >= lk) f(z);
            });
        };
        const float tp_val = key_val<LOW>(radix_select<true, LOW>(kept, (double)tp * S, mx, c64, sh));
        if (tp_val > theta) {
            theta = tp_val;
            S = fblock_sum<NT>(part_sum(theta), sh);
        }
    }
    theta_out = theta;
    S_out = S;
}

// Record 0 of vector v is rec0, its other records are empty.
template <int NT = kFilterBlock>
__device__ __forceinline__ void write_records(const Params &P, int64_t v, const Partial &rec0)
{
    const int64_t ipv = P.geo.ipv;
    for (int64_t j = tid_now(); j < ipv; j += NT)
        P.parts[v * ipv + j] = j == 0 ? rec0 : Partial{-INFINITY, INT32_MAX, 0.0};
}

// Thresholds of vector v after the streaming pass, reading the vector from memory in
// every pass (1024 threads): for vocabularies beyond filter_units_kernel's budget.
template <int DT, bool AL>
__device__ __forceinline__ void filter_vector(const Params &P, int64_t v, FilterLds &sh)
{
    const int tid = tid_now();
    const VecCtx vc = vec_ctx(P, v);
    const int32_t rm = row_mode(P.mode, vc.T);
    const int64_t k = P.top_k ? P.top_k[vc.row] : 0;
    const float tp = P.top_p ? P.top_p[vc.row] : 1.0f;
    const bool use_k = k > 0 && k < P.V, use_p = tp > 0.0f && tp < 1.0f;
    if (rm != ROW_SAMPLE || (!use_k && !use_p)) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const bool target = v < P.nT;
    const void *base = vec_ptr(target ? P.target : P.draft, DT, target ? v : v - P.nT, P.V);
    const int64_t nunits = (P.V + kUnitElems - 1) / kUnitElems;
    const void *arr = target ? P.target : P.draft;
    const uint64_t arr_bytes = (uint64_t)(target ? P.nT : P.nD) * (uint64_t)P.V * (DT == 0 ? 2u : 4u);

    // the maximum (NaN if any logit is); NaN, +inf or no finite logit leaves the
    // vector unfiltered (its row is reported non-finite)
    float tmx = -INFINITY;
    each_logit<DT, AL>(base, P.V, nunits, arr, arr_bytes, [&](float z) { tmx = nmax(tmx, z); });
    const float mx = block_nmax(tmx, sh);
    if (!(mx > -INFINITY && mx < INFINITY)) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const double c64 = kLog2e / (double)vc.T;
    auto from_hbm = [&](auto &&f) { each_logit<DT, AL>(base, P.V, nunits, arr, arr_bytes, f); };
    auto gather_ge = [&](float L, auto &&f) {
        from_hbm([&](float z) {
            if (z >= L) f(z);
        });
    };
    auto part_sum = [&](float lower) {
        double s = 0.0;
        from_hbm([&](float z) {
            if (z >= lower) s += fexp2(((double)z - (double)mx) * c64);
        });
        return s;
    };
    float theta;
    double S;
    constexpr int LOW = DT == 0 ? 16 : 0;
    const uint32_t ncand = gather_candidates<LOW>(gather_ge, tmx, mx, k, use_k, c64, sh);
    finish_thresholds<LOW>(from_hbm, part_sum, ncand, mx, k, tp, use_k, use_p, c64, sh, theta, S);
    write_records(P, v, Partial{mx, __float_as_int(__builtin_nanf("")), S});
    if (tid == 0) {
        P.theta[v] = theta;
        if (vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V) {
            float *zx = P.zx + (target ? 0 : P.nD) + vc.slot;
            const float zv = *zx;
            if (zv < theta) *zx = -INFINITY;
        }
    }
}

// One workgroup per vector.
template <int DT, bool AL>
__global__ __launch_bounds__(kFilterBlock) void filter_kernel(Params P)
{
    __shared__ FilterLds sh;
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    filter_vector<DT, AL>(P, blockIdx.x, sh);
}

// ---------------------------------------------------------------------------
// Thresholds after a streaming pass that stored the maximum of every unit of 64
// consecutive logits (umax, as 16-bit keys; each maximum a different logit).  With
// top-k, any value that k unit maxima reach is a lower bound L of theta_k, so only
// the units whose maximum reaches L are read again (one 128-byte line per bf16
// unit), and the selects run on their logits >= L in LDS.  L as in the other
// kernels, from maxima over the threads: each wave's m-th largest lane maximum
// (m = ceil(k / waves); a lane maximum covers the lane's units), and L their least
// (a block-wide select over all unit maxima when fewer waves hold m finite lanes).
// Rows without top-k, or whose candidates do not fit, take the selects over the
// whole vector.  One two-wave workgroup per vector, 16 per CU: the work is a chain of
// small dependent reads, so many vectors are kept in flight.
// ---------------------------------------------------------------------------
constexpr int kUnitsBlock = 128;
constexpr int kUnitsWaves = kUnitsBlock / 64;
constexpr int kMaxUnitList = 768;   // units read again

// Under 10 KB, so that 16 workgroups fit a CU's LDS.
struct UnitsLds {
    static constexpr uint32_t kCap = 1536;
    float cand[kCap];
    uint32_t ncand;
    union {   // a select's histogram: counts or masses, never both at once
        uint32_t cnt[kBins];
        double mass[kBins];
    };
    double rd[kUnitsWaves];
    float rf[kUnitsWaves];
    uint32_t ru[kUnitsWaves];
    uint32_t rL[kUnitsWaves];
    uint32_t rsel;
    double rabove;
    float wtheta;
    double wS;
    uint32_t nlist;
    uint16_t list[kMaxUnitList];
};
static_assert(sizeof(UnitsLds) <= 10240, "16 select workgroups per CU");

// NUM: units per thread, a multiple of 8 (the vector's ipv * 64 units, at most
// NUM * kUnitsBlock); thread t holds units 8 (t + q NT) + i, i < 8, read 16 bytes at a
// time.
template <int DT, bool AL, int NUM>
__global__ __launch_bounds__(kUnitsBlock) void filter_units_kernel(Params P)
{
    constexpr int NT = kUnitsBlock;
    constexpr int E = DT == 0 ? 8 : 4;                  // logits per 16 bytes
    constexpr int kChunks = kPieceUnits / E;            // 16-byte chunks of a unit
    constexpr int LOW = DT == 0 ? 16 : 0;
    constexpr uint32_t kBad = 0xffff0000u;              // a NaN or +inf unit maximum
    __shared__ UnitsLds sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t v = blockIdx.x;
    // the thread's units: keys in the upper half-word, 0 for -inf (loaded first, so
    // that the row's context loads overlap them)
    const int32_t nu = (int32_t)(P.geo.ipv * kPieceUnits);   // a multiple of 64
    const uint4 *um = reinterpret_cast<const uint4 *>(P.umax + v * (int64_t)nu);
    // (two to a word: key(i) unpacks unit i's)
    uint32_t kw[NUM / 2];
#pragma unroll
    for (int q = 0; q < NUM / 8; ++q) {
        const int32_t g = tid + q * NT;
        const uint4 w = 8 * g < nu ? um[g] : make_uint4(0u, 0u, 0u, 0u);
        kw[4 * q] = w.x;
        kw[4 * q + 1] = w.y;
        kw[4 * q + 2] = w.z;
        kw[4 * q + 3] = w.w;
    }
    auto key = [&](int i) __attribute__((always_inline)) -> uint32_t {
        return (i & 1) ? (kw[i / 2] & 0xffff0000u) : (kw[i / 2] << 16);
    };
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const VecCtx vc = vec_ctx_uniform(P, v);
    const int32_t rm = row_mode(P.mode, vc.T);
    const int64_t k = P.top_k ? load_uniform(P.top_k, vc.row) : 0;
    const float tp = P.top_p ? load_uniform(P.top_p, vc.row) : 1.0f;
    const bool use_k = k > 0 && k < P.V, use_p = tp > 0.0f && tp < 1.0f;
    if (rm != ROW_SAMPLE || (!use_k && !use_p)) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const bool target = v < P.nT;
    const void *arr = target ? P.target : P.draft;
    const void *base = vec_ptr(arr, DT, target ? v : v - P.nT, P.V);
    const int64_t nunits = (P.V + kUnitElems - 1) / kUnitElems;
    const uint64_t arr_bytes = (uint64_t)(target ? P.nT : P.nD) * (uint64_t)P.V * (DT == 0 ? 2u : 4u);

    // per wave, in one barrier: a non-finite maximum, the finite units, and with top-k
    // the m-th largest lane maximum (lanes hold different units, so m lanes whose
    // maximum reaches it hold m logits >= it)
    const int64_t m = use_k ? (k + kUnitsWaves - 1) / kUnitsWaves : 0;
    {
        bool bad = false;
        int wf = 0;
        uint32_t kmax = 0u;
#pragma unroll
        for (int i = 0; i < NUM; ++i) {
            const uint32_t ki = key(i);
            bad |= ki == kBad;
            wf += __popcll(__ballot(ki != 0u));
            kmax = ki > kmax ? ki : kmax;
        }
        uint32_t Lw = 0xffffffffu;   // none
        if (m > 0 && m <= 64 && __popcll(__ballot(kmax != 0u)) >= m) {
            const uint32_t lk[1] = {kmax};
            Lw = wave_select_count<16, 1>(lk, m);
        }
        const bool wbad = __any(bad);
        if (lane == 0) {
            sh.ru[wave] = (uint32_t)wf | (wbad ? 0x80000000u : 0u);
            sh.rL[wave] = Lw;
        }
        if (tid == 0) {
            sh.nlist = 0u;
            sh.ncand = 0u;
        }
    }
    // later uses unpack the keys again from their words, rather than keep them
    // unpacked across the barrier
#pragma unroll
    for (int i = 0; i < NUM / 2; ++i) asm volatile("" : "+v"(kw[i]));
    __syncthreads();
    int64_t nfin = 0;
    bool bad = false;
    uint32_t L32 = 0xffffffffu;
    int nw = 0;
#pragma unroll
    for (int w = 0; w < kUnitsWaves; ++w) {
        const uint32_t r = sh.ru[w];
        bad |= (r & 0x80000000u) != 0u;
        nfin += (int64_t)(r & 0x7fffffffu);
        const uint32_t lw = sh.rL[w];
        if (lw != 0xffffffffu) {
            L32 = lw < L32 ? lw : L32;
            ++nw;
        }
    }
    // a NaN or +inf logit (the row is reported non-finite) or no finite logit: the
    // vector stays unfiltered
    if (bad || nfin == 0) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const double c64 = kLog2e / (double)vc.T;
    uint32_t ncand = kNoCand;
    float mx = -INFINITY;
    if (use_k && k <= nfin) {
        if ((int64_t)nw * m < k) {
            auto from_keys = [&](auto &&f) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < NUM; ++i)
                    if (key(i) != 0u) f(key_val<0>(key(i)));
            };
            L32 = radix_select<false, 16>(from_keys, (double)k, 0.0f, c64, sh);
        }
        // the units whose maximum reaches L
#pragma unroll
        for (int i = 0; i < NUM; ++i) {
            if (key(i) >= L32) {
                const uint32_t at = atomicAdd(&sh.nlist, 1u);
                if (at < (uint32_t)kMaxUnitList) sh.list[at] = (uint16_t)(8 * (tid + (i / 8) * NT) + i % 8);
            }
        }
        __syncthreads();
        const uint32_t nlist = sh.nlist;
        if (nlist <= (uint32_t)kMaxUnitList) {
            // their logits >= L (L the least float of its key, so a lower bound for
            // fp32 maxima rounded down to 16 bits, exact for bf16), eight 16-byte chunks
            // per thread in flight (consecutive threads read consecutive chunks)
            constexpr int kQ = 8;
            const float L = key_val<0>(L32);
            const int32_t nch = (int32_t)nlist * kChunks;
            float tmx = -INFINITY;
            for (int32_t c0 = 0; c0 < nch; c0 += kQ * NT) {
                uint32_t w[kQ][4];
                int32_t e0[kQ];   // (V < 2^31)
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const int32_t c = c0 + q * NT + tid;
                    e0[q] = (int32_t)P.V;   // nothing to read
                    if (c < nch) e0[q] = (int32_t)sh.list[c / kChunks] * kPieceUnits + (c % kChunks) * E;
                    if (e0[q] < P.V) {
                        if constexpr (AL) {
                            const uint4 x = *reinterpret_cast<const uint4 *>(
                                static_cast<const char *>(base) + e0[q] * (DT == 0 ? 2 : 4));
                            w[q][0] = x.x; w[q][1] = x.y; w[q][2] = x.z; w[q][3] = x.w;
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    if (!(e0[q] < P.V)) continue;
#pragma unroll
                    for (int t = 0; t < E; ++t) {
                        float z;
                        if constexpr (AL) {
                            z = DT == 0 ? ((t & 1) ? bf16_hi(w[q][t / 2]) : bf16_lo(w[q][t / 2]))
                                        : __uint_as_float(w[q][t]);
                        } else {
                            if (e0[q] + t >= P.V) break;
                            z = load_logit<DT>(base, e0[q] + t);
                        }
                        if (z >= L) {
                            const uint32_t at = atomicAdd(&sh.ncand, 1u);
                            if (at < UnitsLds::kCap) sh.cand[at] = z;
                            tmx = nmax(tmx, z);
                        }
                    }
                }
            }
            // the maximum is among them
            tmx = wave_umax_f32(tmx);
            if (lane == 0) sh.rf[wave] = tmx;
            __syncthreads();
            ncand = sh.ncand;
#pragma unroll
            for (int w = 0; w < kUnitsWaves; ++w) mx = nmax(mx, sh.rf[w]);
        }
    }
    auto from_hbm = [&](auto &&f) { each_logit<DT, AL, NT>(base, P.V, nunits, arr, arr_bytes, f); };
    if (ncand == kNoCand || ncand > UnitsLds::kCap) {
        // the selects over the whole vector: its maximum first
        float t = -INFINITY;
        from_hbm([&](float z) { t = nmax(t, z); });
        mx = block_nmax<NT>(t, sh);
    }
    auto part_sum = [&](float lower) {
        double s = 0.0;
        from_hbm([&](float z) {
            if (z >= lower) s += fexp2(((double)z - (double)mx) * c64);
        });
        return s;
    };
    float theta;
    double S;
    finish_thresholds<LOW, NT>(from_hbm, part_sum, ncand, mx, k, tp, use_k, use_p, c64, sh, theta, S);
    write_records<NT>(P, v, Partial{mx, __float_as_int(__builtin_nanf("")), S});
    if (tid == 0) {
        P.theta[v] = theta;
        if (vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V) {
            float *zx = P.zx + (target ? 0 : P.nD) + vc.slot;
            const float zv = *zx;
            if (zv < theta) *zx = -INFINITY;
        }
    }
}

hipError_t launch_filter(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const int64_t nvec = P.nT + P.nD;
    if (nvec <= 0) return hipSuccess;
    if (nvec > INT32_MAX) return hipErrorInvalidConfiguration;
    const void *fn = dtype == 0
        ? (aligned ? (const void *)filter_kernel<0, true> : (const void *)filter_kernel<0, false>)
        : (aligned ? (const void *)filter_kernel<1, true> : (const void *)filter_kernel<1, false>);
    void *args[] = {const_cast<Params *>(&P)};
    return hipLaunchKernel(fn, dim3((unsigned)nvec), dim3(kFilterBlock), args, 0, s);
}

// Units per thread of filter_units_kernel for a vocabulary, 0 beyond what it holds.
int filter_units_num(int64_t V)
{
    const int64_t nu = ceil_div(V, 2 * kItemElems) * kPieceUnits;
    for (int n : {8, 16, 24, 32, 64})
        if (nu <= (int64_t)n * kUnitsBlock) return n;
    return 0;
}

template <int DT, bool AL>
static const void *filter_units_fn(int num)
{
    switch (num) {
    case 8: return (const void *)filter_units_kernel<DT, AL, 8>;
    case 16: return (const void *)filter_units_kernel<DT, AL, 16>;
    case 24: return (const void *)filter_units_kernel<DT, AL, 24>;
    case 32: return (const void *)filter_units_kernel<DT, AL, 32>;
    case 64: return (const void *)filter_units_kernel<DT, AL, 64>;
    default: return nullptr;
    }
}

hipError_t launch_filter_units(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const int64_t nvec = P.nT + P.nD;
    if (nvec <= 0) return hipSuccess;
    if (nvec > INT32_MAX || P.umax == nullptr) return hipErrorInvalidConfiguration;
    const int num = filter_units_num(P.V);
    const void *fn = dtype == 0 ? (aligned ? filter_units_fn<0, true>(num) : filter_units_fn<0, false>(num))
                                : (aligned ? filter_units_fn<1, true>(num) : filter_units_fn<1, false>(num));
    if (fn == nullptr) return hipErrorInvalidValue;
    void *args[] = {const_cast<Params *>(&P)};
    return hipLaunchKernel(fn, dim3((unsigned)nvec), dim3(kUnitsBlock), args, 0, s);
}

}  // namespace sv
