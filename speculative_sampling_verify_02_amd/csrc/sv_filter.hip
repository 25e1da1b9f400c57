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
// filter_kernel runs one workgroup of 1024 threads per vector whose row filters.  With
// top-k (k <= 1024) the k-th largest of the threads' maxima bounds theta_k from below;
// the logits above that bound are gathered in LDS (usually little more than k) and
// every later search runs there, so the vector is read twice.  Otherwise a threshold
// is found on the vector itself.  A threshold is found by a bucket search over the
// logit values: 256 buckets of equal
// width over the current value range [lo, hi] take the count (top-k) or the fp64
// probability mass (top-p, exp at the exact scale log2(e)/T) of their logits in LDS;
// the bucket where the running total from the top reaches the target becomes the
// next range, narrowed to its smallest and largest logit, until one value remains.
// Every level reads the vector once (bucket index (hi - z)/width is monotone in z,
// so buckets are value intervals).  The vector's statistics record is then replaced
// by the filtered one (maximum, exact sum over the kept tokens) and the logit at the
// position's draft token is dropped when it falls below theta.
#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

constexpr int kFilterBlock = 1024;
constexpr int kFilterWaves = kFilterBlock / 64;
constexpr int kBins = 256;

// A finite or infinite float as an unsigned key that sorts like the float.
__device__ __forceinline__ uint32_t fkey(float x)
{
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float fkey_val(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kMaxCand = 4096;   // logits kept in LDS by the top-k candidate path

struct FilterLds {
    float tmax[kFilterBlock];        // per-thread maxima
    float cand[kMaxCand];            // logits at or above a lower bound of theta_k
    uint32_t ncand;
    uint32_t cnt[kBins];
    double mass[kBins];
    uint32_t kmin[kBins], kmax[kBins];
    double rd[kFilterWaves];
    float rf[kFilterWaves][2];
    uint32_t ru[kFilterWaves];
    int32_t sel;
    double sel_above;
};

__device__ __forceinline__ double fblock_sum(double v, FilterLds &sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

// Every logit of the vector through f(z), 8 per thread per step.
template <int DT, bool AL, class F>
__device__ __forceinline__ void each_logit(const void *base, int64_t V, int64_t nunits, F &&f)
{
    for (int64_t u = threadIdx.x; u < nunits; u += kFilterBlock) {
        const RawUnit<DT> r = load_raw<DT, AL>(base, u, V);
        float z[kUnitElems];
        unpack<DT>(r, z);
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) f(z[e]);
    }
}

// The largest logit value t in [lo, hi] whose metric over {z >= t} reaches target,
// where `above` is the metric over {z > hi} (count, or fp64 mass 2^((z - m) c64)).
template <bool MASS, class Src>
__device__ __forceinline__ float bucket_search(Src &&each, float lo, float hi, double above, double target, float m, double c64,
                               FilterLds &sh)
{
    const int tid = threadIdx.x, lane = tid & 63;
    for (int level = 0; level < 64; ++level) {   // each level leaves fewer distinct values
        if (!(lo < hi)) break;
        const float width = (hi - lo) * (1.0f / kBins);
        const float inv_w = 1.0f / width;
        if (tid < kBins) {
            sh.cnt[tid] = 0u;
            sh.mass[tid] = 0.0;
            sh.kmin[tid] = 0xffffffffu;
            sh.kmax[tid] = 0u;
        }
        __syncthreads();
        each([&](float z) __attribute__((always_inline)) {
            if (z >= lo && z <= hi) {
                const float q = (hi - z) * inv_w;   // NaN only for z == hi with width 0
                const int d = q != q ? 0 : (q >= (float)(kBins - 1) ? kBins - 1 : (int)q);
                atomicAdd(&sh.cnt[d], 1u);
                if constexpr (MASS) atomicAdd(&sh.mass[d], exp2_f64(((double)z - (double)m) * c64));
                atomicMin(&sh.kmin[d], fkey(z));
                atomicMax(&sh.kmax[d], fkey(z));
            }
        });
        __syncthreads();
        if (tid < 64) {
            // four bins per lane, in order; the first bin where the running total
            // reaches the target (else the last non-empty one)
            double v[4], lsum = 0.0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = lane * 4 + k;
                v[k] = MASS ? sh.mass[d] : (double)sh.cnt[d];
                lsum += v[k];
            }
            const double incl = wave_inclusive_sum(lsum, lane);
            double run = above + incl - lsum;
            int hit = -1, lastne = -1;
            double hit_before = 0.0, last_before = 0.0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = lane * 4 + k;
                if (hit < 0 && run + v[k] >= target && sh.cnt[d] > 0u) { hit = d; hit_before = run; }
                if (sh.cnt[d] > 0u) { lastne = d; last_before = run; }
                run += v[k];
            }
            const unsigned long long hb = __ballot(hit >= 0);
            int dsel;
            double before;
            if (hb) {
                const int l = __ffsll((long long)hb) - 1;
                dsel = __shfl(hit, l);
                before = __shfl(hit_before, l);
            } else {
                const unsigned long long nb = __ballot(lastne >= 0);
                const int l = nb ? 63 - __clzll((long long)nb) : 0;
                dsel = nb ? __shfl(lastne, l) : 0;
                before = nb ? __shfl(last_before, l) : above;
            }
            if (lane == 0) {
                sh.sel = dsel;
                sh.sel_above = before;
            }
        }
        __syncthreads();
        const int d = sh.sel;
        above = sh.sel_above;
        const float nlo = fkey_val(sh.kmin[d]), nhi = fkey_val(sh.kmax[d]);
        __syncthreads();
        lo = nlo;
        hi = nhi;
    }
    return hi;
}

// Block-wide maximum of the threads' values, NaN if any is NaN.
__device__ __forceinline__ float block_nmax(float v, FilterLds &sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_umax_f32(v);
    if (lane == 0) sh.rf[wave][0] = v;
    __syncthreads();
    float m = -INFINITY;
    for (int w = 0; w < kFilterWaves; ++w) m = nmax(m, sh.rf[w][0]);
    __syncthreads();
    return m;
}

// Block-wide minimum of the threads' values (no NaN among them).
__device__ __forceinline__ float block_min(float v, FilterLds &sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    if (lane == 0) sh.rf[wave][1] = v;
    __syncthreads();
    float m = INFINITY;
    for (int w = 0; w < kFilterWaves; ++w) m = fminf(m, sh.rf[w][1]);
    __syncthreads();
    return m;
}

// theta = max(theta_k, theta_p) of one vector whose logits are finite or -inf, with
// maximum mx > -inf, and the fp64 sum over the kept logits of 2^((z - mx) c64).
// `gather(f)` and `each(f)` both pass every logit of the vector to f (spread over
// the threads, any order): the first once, to gather top-k candidates, the second
// for the searches over the whole vector; `part_sum(lower)` is this thread's share
// of the sum over the logits >= lower.  tmx is this thread's maximum under `gather`.
template <class Gather, class Each, class PartSum>
__device__ __forceinline__ void thresholds(Gather &&gather, Each &&each, PartSum &&part_sum, float tmx, float mx,
                                           int64_t k, float tp, bool use_k, bool use_p, double c64, FilterLds &sh,
                                           float &theta_out, double &S_out)
{
    const int tid = threadIdx.x;
    auto from_cand = [&](auto &&f) {
        for (uint32_t i = tid; i < sh.ncand; i += kFilterBlock) f(sh.cand[i]);
    };
    float theta = -INFINITY;
    double S = 0.0;
    bool in_lds = false;
    float L = -INFINITY;
    // threads whose maximum is finite (each such maximum is a different logit)
    const int nmax_fin = __syncthreads_count(tmx > -INFINITY);
    if (use_k && k <= nmax_fin) {
        // top-k candidates: the k-th largest of the per-thread maxima is a lower bound L
        // of theta_k (those maxima are logits of the vector); the logits >= L, at
        // least k of them, usually fit in LDS and every later step runs there
        const float tlo = block_min(tmx > -INFINITY ? tmx : INFINITY, sh);
        sh.tmax[tid] = tmx;
        if (tid == 0) sh.ncand = 0u;
        __syncthreads();
        auto from_tmax = [&](auto &&f) { f(sh.tmax[tid]); };
        L = bucket_search<false>(from_tmax, tlo, mx, 0.0, (double)k, mx, c64, sh);
        if (tmx >= L) {   // only threads holding a logit >= L
            gather([&](float z) __attribute__((always_inline)) {
                if (z >= L) {
                    const uint32_t i = atomicAdd(&sh.ncand, 1u);
                    if (i < (uint32_t)kMaxCand) sh.cand[i] = z;
                }
            });
        }
        __syncthreads();
        in_lds = sh.ncand <= (uint32_t)kMaxCand;
    }
    if (in_lds) {
        theta = bucket_search<false>(from_cand, L, mx, 0.0, (double)k, mx, c64, sh);
        if (use_p) {
            const float lower = theta;
            double s = 0.0;
            from_cand([&](float z) {
                if (z >= lower) s += exp2_f64(((double)z - (double)mx) * c64);
            });
            const double Sk = fblock_sum(s, sh);
            theta = fmaxf(theta, bucket_search<true>(from_cand, lower, mx, 0.0, (double)tp * Sk, mx, c64, sh));
        }
        double s = 0.0;
        from_cand([&](float z) {
            if (z >= theta) s += exp2_f64(((double)z - (double)mx) * c64);
        });
        S = fblock_sum(s, sh);
    } else {
        // searches over the whole vector: its smallest finite logit and finite count first
        float mn = INFINITY;
        uint32_t nfin = 0u;
        each([&](float z) {
            if (z > -INFINITY) {
                mn = fminf(mn, z);
                ++nfin;
            }
        });
        mn = block_min(mn, sh);
        nfin = (uint32_t)fblock_sum((double)nfin, sh);
        if (use_k && (uint64_t)k <= nfin) theta = bucket_search<false>(each, mn, mx, 0.0, (double)k, mx, c64, sh);
        if (use_p) {
            const float lower = theta > -INFINITY ? theta : mn;
            const double Sk = fblock_sum(part_sum(lower), sh);
            theta = fmaxf(theta, bucket_search<true>(each, lower, mx, 0.0, (double)tp * Sk, mx, c64, sh));
        }
        S = fblock_sum(part_sum(theta), sh);
    }
    theta_out = theta;
    S_out = S;
}

// Record 0 of vector v is rec0, its other records are empty.
__device__ __forceinline__ void write_records(const Params &P, int64_t v, const Partial &rec0)
{
    const int64_t ipv = P.geo.ipv;
    for (int64_t j = threadIdx.x; j < ipv; j += kFilterBlock)
        P.parts[v * ipv + j] = j == 0 ? rec0 : Partial{-INFINITY, INT32_MAX, 0.0};
}

// Thresholds after the streaming pass (fp32 logits, rows that are not 16-byte
// aligned, vocabularies beyond what filter_stats_kernel holds in registers): the
// vector is read from memory by every pass.
template <int DT, bool AL>
__global__ __launch_bounds__(kFilterBlock) void filter_kernel(Params P)
{
    __shared__ FilterLds sh;
    const int tid = threadIdx.x;
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

    // the maximum (NaN if any logit is); NaN, +inf or no finite logit leaves the
    // vector unfiltered (its row is reported non-finite)
    float tmx = -INFINITY;
    each_logit<DT, AL>(base, P.V, nunits, [&](float z) { tmx = nmax(tmx, z); });
    const float mx = block_nmax(tmx, sh);
    if (!(mx > -INFINITY && mx < INFINITY)) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const double c64 = kLog2e / (double)vc.T;
    auto from_hbm = [&](auto &&f) { each_logit<DT, AL>(base, P.V, nunits, f); };
    auto part_sum = [&](float lower) {
        double s = 0.0;
        from_hbm([&](float z) {
            if (z >= lower) s += exp2_f64(((double)z - (double)mx) * c64);
        });
        return s;
    };
    float theta;
    double S;
    thresholds(from_hbm, from_hbm, part_sum, tmx, mx, k, tp, use_k, use_p, c64, sh, theta, S);
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

// The raw words of a unit as the compiler must assume them changed: a pass over the
// register-resident vector unpacks its logits where it uses them, instead of keeping
// the unpacked values of every unit live across passes.
__device__ __forceinline__ void opaque(uint32_t (&w)[4])
{
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
}

template <int NU>
__global__ __launch_bounds__(kFilterBlock) void filter_stats_kernel(Params P)
{
    __shared__ FilterLds sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t v = blockIdx.x;
    const bool target = v < P.nT;
    const uint16_t *base =
        static_cast<const uint16_t *>(vec_ptr(target ? P.target : P.draft, 0, target ? v : v - P.nT, P.V));
    const int32_t nunits = (int32_t)(P.V / kUnitElems);   // aligned rows: V is a multiple of 8
    // every load of the vector first, unconditional (a unit past the end reads the
    // last unit and becomes -inf once loaded)
    uint4 r[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int32_t u = tid + i * kFilterBlock;
        r[i] = reinterpret_cast<const uint4 *>(base)[u < nunits ? u : nunits - 1];
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
        opaque(w);
        const bool in = tid + i * kFilterBlock < nunits;
        r[i] = in ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const VecCtx vc = vec_ctx(P, v);
    const bool has_x = vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V;
    const float zx = (tid == 0 && has_x) ? load_logit<0>(base, vc.x) : -INFINITY;
    const int32_t rm = row_mode(P.mode, vc.T);

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
    auto each = [&](auto &&f) __attribute__((always_inline)) {
        each_idx([&](float z, int32_t) __attribute__((always_inline)) { f(z); });
    };

    // the maximum, NaN if any logit is
    float tmx = -INFINITY;
    each([&](float z) __attribute__((always_inline)) { tmx = nmax(tmx, z); });
    const float mx = block_nmax(tmx, sh);

    if (rm != ROW_SAMPLE) {
        // greedy rows: the target vectors' first argmax (NaN: no index); bad
        // temperatures: nothing
        Partial rec{-INFINITY, INT32_MAX, 0.0};
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
        write_records(P, v, rec);
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }

    float theta = -INFINITY;
    Partial rec{mx, __float_as_int(__builtin_nanf("")), 0.0};
    if (!(mx < INFINITY)) {
        // a NaN or +inf logit: the row is reported non-finite
        rec.s = (double)__builtin_nanf("");
    } else if (mx == -INFINITY) {
        rec = Partial{-INFINITY, 0, 0.0};
    } else {
        const double c64 = kLog2e / (double)vc.T;
        const float c32 = (float)c64;
        const int64_t k = P.top_k ? P.top_k[vc.row] : 0;
        const float tp = P.top_p ? P.top_p[vc.row] : 1.0f;
        const bool use_k = k > 0 && k < P.V, use_p = tp > 0.0f && tp < 1.0f;
        double S;
        if (use_k || use_p) {
            // searches that do not run on top-k candidates in LDS read the vector from
            // memory again, in fp64 like filter_kernel (the vector's registers are
            // free by then)
            auto from_hbm = [&](auto &&f) { each_logit<0, true>(base, P.V, nunits, f); };
            auto part_sum = [&](float lower) {
                double s = 0.0;
                from_hbm([&](float z) {
                    if (z >= lower) s += exp2_f64(((double)z - (double)mx) * c64);
                });
                return s;
            };
            thresholds(each, from_hbm, part_sum, tmx, mx, k, tp, use_k, use_p, c64, sh, theta, S);
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
        rec.s = S;
    }
    write_records(P, v, rec);
    if (tid == 0) {
        P.theta[v] = theta;
        if (has_x) P.zx[(target ? 0 : P.nD) + vc.slot] = zx < theta ? -INFINITY : zx;
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

// Units per thread of filter_stats_kernel for this call, 0 when it does not apply.
int filter_stats_units(int dtype, bool aligned, int64_t V)
{
    if (dtype != 0 || !aligned) return 0;
    const int64_t per = (V / kUnitElems + kFilterBlock - 1) / kFilterBlock;
    for (int nu : {4, 8, 12, 16, 20})
        if (per <= nu) return nu;
    return 0;
}

hipError_t launch_filter_stats(const Params &P, hipStream_t s, int nu)
{
    const int64_t nvec = P.nT + P.nD;
    if (nvec <= 0) return hipSuccess;
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
    void *args[] = {const_cast<Params *>(&P)};
    return hipLaunchKernel(fn, dim3((unsigned)nvec), dim3(kFilterBlock), args, 0, s);
}

}  // namespace sv
