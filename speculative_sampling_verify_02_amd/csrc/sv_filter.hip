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
// With top-k (k at most the number of threads holding a finite logit) a lower bound
// L of theta_k comes from the threads' own maxima (per wave, with ballots); the
// logits >= L, at least k of them and usually a few times k, are gathered in LDS and
// every later select runs there, in one wave when they are at most 256 (the same
// selects a key bit at a time, with ballots).  Otherwise the selects run over the
// whole vector.
//
// filter_stats_kernel (16-byte-aligned bf16 rows of up to 163840 logits) holds the
// vector in registers and produces the vector's statistics record, theta and the
// logit at the position's draft token in one pass; filter_kernel runs after the
// streaming pass otherwise, reading the vector from memory in every pass, and
// replaces the record of each vector that filters.
#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

constexpr int kFilterBlock = 1024;
constexpr int kFilterWaves = kFilterBlock / 64;
constexpr int kBins = 256;       // one 8-bit digit
constexpr int kMaxCand = 4096;   // logits kept in LDS by the top-k candidate path

// The thread index as a value the compiler must take as new at every call: what the
// helpers derive from it (lane, wave, LDS offsets) is recomputed where used, not kept
// in registers across the loop of filter_stats_kernel.
__device__ __forceinline__ int tid_now()
{
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// 2^x in fp64 (exp2_f64) with the series' coefficients read from constant memory:
// scalar registers, rather than vector registers held across the loop of
// filter_stats_kernel.
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
    float cand[kMaxCand];   // logits at or above a lower bound of theta_k
    uint32_t ncand;
    uint32_t cnt[kBins];
    double mass[kBins];
    double rd[kFilterWaves];
    float rf[kFilterWaves];
    uint32_t ru[kFilterWaves];
    float rL[kFilterWaves];
    uint32_t rsel;          // radix select: key prefix so far
    double rabove;          // and the metric above it
    float wtheta;           // one-wave select results
    double wS;
};

__device__ __forceinline__ double fblock_sum(double v, FilterLds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) sh.rd[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kFilterWaves; ++w) t += sh.rd[w];
    return t;
}

// Block-wide maximum of the threads' values, NaN if any is NaN.
__device__ __forceinline__ float block_nmax(float v, FilterLds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    v = wave_umax_f32(v);
    if (lane == 0) sh.rf[wave] = v;
    __syncthreads();
    float m = -INFINITY;
    for (int w = 0; w < kFilterWaves; ++w) m = nmax(m, sh.rf[w]);
    __syncthreads();
    return m;
}

// Every logit of the vector through f(z), 8 per thread per step.  Rows that are not
// 16-byte aligned are read a 512-logit tile per wave with aligned loads shifted into
// place (load_tile_unit), the logits past V as -inf (arr, arr_bytes: the array the
// row lies in).
template <int DT, bool AL, class F>
__device__ __forceinline__ void each_logit(const void *base, int64_t V, int64_t nunits, const void *arr,
                                           uint64_t arr_bytes, F &&f)
{
    if constexpr (AL) {
        for (int64_t u = tid_now(); u < nunits; u += kFilterBlock) {
            const RawUnit<DT> r = load_raw<DT, AL>(base, u, V);
            float z[kUnitElems];
            unpack<DT>(r, z);
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) f(z[e]);
        }
    } else {
        const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
        for (int64_t tile = wave; tile * kTileUnits < nunits; tile += kFilterWaves) {
            const RawUnit<DT> r = load_tile_unit<DT>(base, tile, V, arr, arr_bytes, lane);
            float z[kUnitElems];
            unpack<DT>(r, z);
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) f(z[e]);
        }
    }
}

// The largest key t (bits >= LOW) whose metric over {key >= t} reaches target > 0:
// the count of the logits `each` passes (MASS false), or the sum of their weights
// 2^((z - m) c64) (MASS true).  The total metric must reach the target.
template <bool MASS, int LOW, class Src>
__device__ __forceinline__ uint32_t radix_select(Src &&each, double target, float m, double c64, FilterLds &sh)
{
    const int tid = tid_now(), lane = tid & 63;
    uint32_t prefix = 0u;
    double above = 0.0;
#pragma unroll
    for (int shift = 24; shift >= LOW; shift -= 8) {
        if (tid < kBins) {
            if constexpr (MASS) sh.mass[tid] = 0.0;
            else sh.cnt[tid] = 0u;
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
template <int LOW>
__device__ __forceinline__ void one_wave_thresholds(uint32_t ncand, float mx, int64_t k, float tp, bool use_p,
                                                    double c64, FilterLds &sh, float &theta_out, double &S_out)
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
template <int LOW, class Each, class PartSum>
__device__ __forceinline__ void finish_thresholds(Each &&each, PartSum &&part_sum, uint32_t ncand, float mx,
                                                  int64_t k, float tp, bool use_k, bool use_p, double c64,
                                                  FilterLds &sh, float &theta_out, double &S_out)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    if (ncand != kNoCand) {
        if (ncand <= (uint32_t)(kWaveCand * 64)) {
            one_wave_thresholds<LOW>(ncand, mx, k, tp, use_p, c64, sh, theta_out, S_out);
            return;
        }
        if (ncand <= (uint32_t)kMaxCand) {
            auto from_cand = [&](auto &&f) __attribute__((always_inline)) {
                for (uint32_t i = tid; i < ncand; i += kFilterBlock) f(sh.cand[i]);
            };
            float theta = key_val<LOW>(radix_select<false, LOW>(from_cand, (double)k, mx, c64, sh));
            auto cand_sum = [&](float lower) {
                double s = 0.0;
                from_cand([&](float z) {
                    if (z >= lower) s += fexp2(((double)z - (double)mx) * c64);
                });
                return fblock_sum(s, sh);
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
            return;
        }
    }
    // selects over the whole vector; theta_k needs at least k finite logits
    uint32_t nfin = 0u;
    each([&](float z) {
        if (z > -INFINITY) ++nfin;
    });
    nfin = (uint32_t)fblock_sum((double)nfin, sh);
    float theta = -INFINITY;
    if (use_k && (uint64_t)k <= nfin) theta = key_val<LOW>(radix_select<false, LOW>(each, (double)k, mx, c64, sh));
    double S = fblock_sum(part_sum(theta), sh);
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
            S = fblock_sum(part_sum(theta), sh);
        }
    }
    theta_out = theta;
    S_out = S;
}

// Record 0 of vector v is rec0, its other records are empty.
__device__ __forceinline__ void write_records(const Params &P, int64_t v, const Partial &rec0)
{
    const int64_t ipv = P.geo.ipv;
    for (int64_t j = tid_now(); j < ipv; j += kFilterBlock)
        P.parts[v * ipv + j] = j == 0 ? rec0 : Partial{-INFINITY, INT32_MAX, 0.0};
}

// Thresholds after the streaming pass (fp32 logits, rows that are not 16-byte
// aligned, vocabularies beyond what filter_stats_kernel holds in registers): the
// vector is read from memory by every pass.
template <int DT, bool AL>
__global__ __launch_bounds__(kFilterBlock) void filter_kernel(Params P)
{
    __shared__ FilterLds sh;
    const int tid = tid_now();
    const int64_t v = blockIdx.x;
    if (P.gamma != nullptr && P.hdr->status != 0) return;
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

// ---------------------------------------------------------------------------
// The whole pass of a filtered call in one kernel, for 16-byte-aligned bf16 rows of
// at most NU * 8192 logits: the workgroup loads its vector once into registers (NU
// 16-byte units per thread) and computes from there what the streaming pass and the
// threshold search compute together otherwise: the vector's record (maximum and sum
// over the kept logits, or the first argmax of a greedy row), theta, and the logit
// at the position's draft token (-inf when it falls below theta).
// ---------------------------------------------------------------------------

// What the register-resident kernel needs from its threads' maxima, in one barrier:
// the block maximum (NaN if any logit is), the number of threads whose maximum is
// finite (each such maximum is a different logit), and, with m > 0, each wave's m-th
// largest finite thread maximum, the least of them being L (nw such waves hold at
// least nw m logits >= L, so L bounds the k-th largest logit from below when
// nw m >= k).  Also clears the candidate count.
struct MaxStats {
    float mx;
    int nfin;
    float L;
    int nw;
};

__device__ __forceinline__ MaxStats block_max_stats(float tmx, int64_t m, FilterLds &sh)
{
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    const float wm = wave_umax_f32(tmx);
    const int wf = __popcll(__ballot(tmx > -INFINITY));
    float Lw = INFINITY;
    if (m > 0 && wf >= m) {
        const uint32_t key[1] = {tmx > -INFINITY ? fkey(tmx) : 0u};
        Lw = key_val<16>(wave_select_count<16, 1>(key, m));
    }
    if (lane == 0) {
        sh.rf[wave] = wm;
        sh.ru[wave] = (uint32_t)wf;
        sh.rL[wave] = Lw;
    }
    if (tid == 0) sh.ncand = 0u;
    __syncthreads();
    MaxStats r{-INFINITY, 0, INFINITY, 0};
    for (int w = 0; w < kFilterWaves; ++w) {
        r.mx = nmax(r.mx, sh.rf[w]);
        r.nfin += (int)sh.ru[w];
        const float lw = sh.rL[w];
        if (lw < INFINITY) {
            r.L = fminf(r.L, lw);
            ++r.nw;
        }
    }
    __syncthreads();   // sh.rf, sh.ru are written again by the greedy argmax
    return r;
}

// The raw words of a unit as the compiler must assume them changed: a pass over the
// register-resident vector unpacks its logits where it uses them, instead of keeping
// the unpacked values of every unit live across passes.
__device__ __forceinline__ void opaque(uint32_t (&w)[4])
{
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
}

// NU units of vector v into registers, every load unconditional (a unit past the end
// reads the last unit); land_vector then waits for them and makes those units -inf.
template <int NU>
__device__ __forceinline__ void load_vector(const Params &P, int64_t v, int32_t nunits, uint4 (&r)[NU])
{
    const bool target = v < P.nT;
    const uint4 *base =
        static_cast<const uint4 *>(vec_ptr(target ? P.target : P.draft, 0, target ? v : v - P.nT, P.V));
    // the lane's unit offsets are recomputed here on every call (32-bit, from a thread
    // index the compiler must take as new), not kept live across the calls
    const uint32_t tid = (uint32_t)tid_now();
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const uint32_t u = tid + (uint32_t)(i * kFilterBlock);
        r[i] = load_nt16(base + (u < (uint32_t)nunits ? u : (uint32_t)nunits - 1u));
    }
}

template <int NU>
__device__ __forceinline__ void land_vector(int32_t nunits, uint4 (&r)[NU], int32_t tid)
{
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
        opaque(w);
        const bool in = tid + i * kFilterBlock < nunits;
        r[i] = in ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
}

// One workgroup per CU takes vectors blockIdx.x, + gridDim.x, ...; the loads of its
// next vector are issued as soon as the current one's registers are no longer read
// (after the top-k gather, usually), so they overlap the rest of its work.
template <int NU>
__global__ __launch_bounds__(kFilterBlock) void filter_stats_kernel(Params P)
{
    __shared__ FilterLds sh;
    // unit maxima of the thread's units beyond what registers hold (two bf16 to a word)
    __shared__ uint32_t s_um[NU > 16 ? (NU + 1) / 2 : 1][kFilterBlock];
    const int tid = tid_now(), lane = tid & 63, wave = tid >> 6;
    const int64_t nvec = P.nT + P.nD;
    const int32_t nunits = (int32_t)(P.V / kUnitElems);   // aligned rows: V is a multiple of 8
    int64_t v = blockIdx.x;
    if (v >= nvec) return;
    uint4 r[NU];
    load_vector<NU>(P, v, nunits, r);
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    for (;;) {
        const int64_t vn = v + gridDim.x;
        const bool has_next = vn < nvec;
        bool issued = false;   // the next vector's loads are in flight
        // the thread index as a new value in every iteration: what derives from it is
        // recomputed where used instead of held in registers across the loop
        const int32_t tid = tid_now();
        land_vector<NU>(nunits, r, tid);
        const bool target = v < P.nT;
        const uint16_t *base =
            static_cast<const uint16_t *>(vec_ptr(target ? P.target : P.draft, 0, target ? v : v - P.nT, P.V));
        // the vector's context, the same on every thread: kept in scalar registers
        VecCtx vc = vec_ctx(P, v);
        vc.row = __builtin_amdgcn_readfirstlane(vc.row);
        vc.slot = __builtin_amdgcn_readfirstlane(vc.slot);
        vc.x = __builtin_amdgcn_readfirstlane(vc.x);
        vc.T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vc.T)));
        const bool has_x = vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V;
        const float zx = (tid == 0 && has_x) ? load_logit<0>(base, vc.x) : -INFINITY;
        const int32_t rm = row_mode(P.mode, vc.T);
        const int64_t k = __builtin_amdgcn_readfirstlane(P.top_k ? P.top_k[vc.row] : 0);
        const float tp =
            __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(P.top_p ? P.top_p[vc.row] : 1.0f)));

        // f(z, i) for every logit z of this thread, i its index in the vector
        auto each_idx = [&](auto &&f) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                opaque(w);
                const int32_t e0 = (tid + i * kFilterBlock) * kUnitElems;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f(bf16_lo(w[t]), e0 + 2 * t);
                    f(bf16_hi(w[t]), e0 + 2 * t + 1);
                }
            }
        };

        // the maximum, NaN if any logit is, and the maximum of every unit (bf16
        // values, two to a word) for the top-k gather: in registers up to 16 units per
        // thread, in LDS beyond (where the registers do not allow)
        constexpr bool kKeepUnitMax = NU <= 16;
        float tmx = -INFINITY;
        uint32_t um2[(NU + 1) / 2];
        uint32_t pend = 0u;   // (LDS) an even unit's maximum, stored with the odd one's
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
            opaque(w);
            float um = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t) um = nmax(um, nmax(bf16_lo(w[t]), bf16_hi(w[t])));
            tmx = nmax(tmx, um);
            const uint32_t ub = __float_as_uint(um) >> 16;
            if constexpr (kKeepUnitMax) {
                if (i & 1) um2[i / 2] |= ub << 16;
                else um2[i / 2] = ub;
            } else {
                if (i & 1) s_um[i / 2][tid] = pend | (ub << 16);
                else pend = ub;
            }
        }
        if constexpr (!kKeepUnitMax && (NU & 1)) s_um[NU / 2][tid] = pend;
        // top-k rows: each wave's m-th largest thread maximum (m = ceil(k / 16)) rides
        // on the maximum's barrier
        const int64_t m = (rm == ROW_SAMPLE && k > 0 && k < P.V) ? (k + kFilterWaves - 1) / kFilterWaves : 0;
        const MaxStats ms = block_max_stats(tmx, m, sh);
        const float mx = ms.mx;

        float theta = -INFINITY;
        Partial rec{-INFINITY, INT32_MAX, 0.0};
        if (rm != ROW_SAMPLE) {
            // greedy rows: the target vectors' first argmax (NaN: no index); bad
            // temperatures: the maximum alone (which tells the row non-finite)
            if (rm == ROW_BAD_TEMP) rec.m = mx;
            if (rm == ROW_GREEDY && target) {
                rec.m = mx;
                if (mx > -INFINITY) {   // not NaN, not -inf
                    int32_t first = INT32_MAX;
                    if (tmx == mx) {
                        each_idx([&](float z, int32_t i) __attribute__((always_inline)) {
                            if (z == mx && i < first) first = i;
                        });
                    }
                    first = wave_umin_i32(first);
                    if (lane == 0) sh.ru[wave] = (uint32_t)first;
                    __syncthreads();
                    for (int w = 0; w < kFilterWaves; ++w) first = min(first, (int32_t)sh.ru[w]);
                    rec.idx = first;
                }
            }
        } else if (!(mx < INFINITY)) {
            // a NaN or +inf logit: the row is reported non-finite
            rec = Partial{mx, __float_as_int(__builtin_nanf("")), (double)__builtin_nanf("")};
        } else if (mx == -INFINITY) {
            rec = Partial{-INFINITY, 0, 0.0};
        } else {
            const double c64 = kLog2e / (double)vc.T;
            const float c32 = (float)c64;
            const bool use_k = k > 0 && k < P.V, use_p = tp > 0.0f && tp < 1.0f;
            double S;
            if (use_k || use_p) {
                // the candidates come from the registers, a unit at a time (units whose
                // maximum is below L are skipped); selects that do not run on
                // candidates in LDS read the vector from memory again, in fp64 like
                // filter_kernel
                auto gather_ge = [&](float L, auto &&f) __attribute__((always_inline)) {
                    if (!(tmx >= L)) return;   // no logit of this thread reaches L
#pragma unroll
                    for (int i = 0; i < NU; ++i) {
                        uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                        opaque(w);
                        float um;
                        if constexpr (kKeepUnitMax) {
                            um = (i & 1) ? bf16_hi(um2[i / 2]) : bf16_lo(um2[i / 2]);
                        } else {
                            const uint32_t uw = s_um[i / 2][tid];
                            um = (i & 1) ? bf16_hi(uw) : bf16_lo(uw);
                        }
                        if (um >= L) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const float zl = bf16_lo(w[t]), zh = bf16_hi(w[t]);
                                if (zl >= L) f(zl);
                                if (zh >= L) f(zh);
                            }
                        }
                    }
                };
                auto from_hbm = [&](auto &&f) { each_logit<0, true>(base, P.V, nunits, nullptr, 0, f); };
                auto part_sum = [&](float lower) {
                    double s = 0.0;
                    from_hbm([&](float z) {
                        if (z >= lower) s += fexp2(((double)z - (double)mx) * c64);
                    });
                    return s;
                };
                // top-k candidates: the logits >= L (fewer waves holding m finite
                // maxima: L is the k-th largest thread maximum, by a block-wide select)
                uint32_t ncand = kNoCand;
                if (use_k && k <= ms.nfin) {
                    float L = ms.L;
                    if ((int64_t)ms.nw * m < k) {
                        auto from_tmax = [&](auto &&f) __attribute__((always_inline)) { f(tmx); };
                        L = key_val<16>(radix_select<false, 16>(from_tmax, (double)k, mx, c64, sh));
                    }
                    gather_ge(L, [&](float z) __attribute__((always_inline)) {
                        const uint32_t i = atomicAdd(&sh.ncand, 1u);
                        if (i < (uint32_t)kMaxCand) sh.cand[i] = z;
                    });
                    __syncthreads();
                    ncand = sh.ncand;
                }
                if (ncand <= (uint32_t)(kWaveCand * 64)) {
                    // the registers are free from here on: the next vector's loads go
                    // out while wave 0 finishes this one (its own loads after, so that
                    // they do not queue ahead of its select)
                    if (has_next && (tid >> 6) != 0) load_vector<NU>(P, vn, nunits, r);
                    one_wave_thresholds<16>(ncand, mx, k, tp, use_p, c64, sh, theta, S);
                    if (has_next && (tid >> 6) == 0) load_vector<NU>(P, vn, nunits, r);
                    issued = true;
                } else {
                    finish_thresholds<16>(from_hbm, part_sum, ncand, mx, k, tp, use_k, use_p, c64, sh, theta, S);
                }
            } else {
                // this thread's sum over all logits: fp32 per unit, fp64 across units
                double s = 0.0;
#pragma unroll
                for (int i = 0; i < NU; ++i) {
                    uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                    opaque(w);
                    float a = 0.0f;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        a += hw_exp2((bf16_lo(w[t]) - mx) * c32);
                        a += hw_exp2((bf16_hi(w[t]) - mx) * c32);
                    }
                    s += (double)a;
                }
                S = fblock_sum(s, sh);
            }
            rec = Partial{mx, __float_as_int(__builtin_nanf("")), S};
        }
        write_records(P, v, rec);
        if (tid == 0) {
            P.theta[v] = theta;
            if (rm == ROW_SAMPLE && has_x) P.zx[(target ? 0 : P.nD) + vc.slot] = zx < theta ? -INFINITY : zx;
        }
        if (!has_next) break;
        if (!issued) load_vector<NU>(P, vn, nunits, r);
        v = vn;
    }
}

// Workgroups of filter_stats_kernel<nu> that fit on the current device at once.
static int32_t filter_grid_cap(const void *fn)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kFilterBlock, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    return cus * per_cu;
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

// Units per thread of filter_stats_kernel for this call, 0 when it does not apply.
int filter_stats_units(int dtype, bool aligned, int64_t V)
{
    if (dtype != 0 || !aligned) return 0;
    const int64_t per = (V / kUnitElems + kFilterBlock - 1) / kFilterBlock;
    for (int nu : {4, 8, 12, 16, 20})
        if (per <= nu) return nu;
    return 0;
}

hipError_t launch_filter_stats(const Params &P, hipStream_t s, int nu, hipEvent_t start, hipEvent_t stop)
{
    const int64_t nvec = P.nT + P.nD;
    if (nvec <= 0) return launch_timed(nullptr, 0, kFilterBlock, P, s, start, stop);
    if (nvec > INT32_MAX) return hipErrorInvalidConfiguration;
    const void *fn = nullptr;
    switch (nu) {
    case 4: fn = (const void *)filter_stats_kernel<4>; break;
    case 8: fn = (const void *)filter_stats_kernel<8>; break;
    case 12: fn = (const void *)filter_stats_kernel<12>; break;
    case 16: fn = (const void *)filter_stats_kernel<16>; break;
    case 20: fn = (const void *)filter_stats_kernel<20>; break;
    default: return hipErrorInvalidValue;
    }
    static int32_t cap[5][64] = {};   // per kernel variant and device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int var = nu / 4 - 1;
    int32_t grid = dev < 64 ? cap[var][dev] : 0;
    if (grid <= 0) {
        grid = filter_grid_cap(fn);
        if (dev < 64) cap[var][dev] = grid;
    }
    const int64_t blocks = nvec < grid ? nvec : grid;
    return launch_timed(fn, blocks, kFilterBlock, P, s, start, stop);
}

}  // namespace sv
