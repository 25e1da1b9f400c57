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
__device__ float bucket_search(Src &&each, float lo, float hi, double above, double target, float m, double c64,
                               FilterLds &sh)
{
    const int tid = threadIdx.x, lane = tid & 63;
    for (int level = 0; level < 64; ++level) {   // each level leaves fewer distinct values
        if (!(lo < hi)) break;
        const float width = (hi - lo) * (1.0f / kBins);
        if (tid < kBins) {
            sh.cnt[tid] = 0u;
            sh.mass[tid] = 0.0;
            sh.kmin[tid] = 0xffffffffu;
            sh.kmax[tid] = 0u;
        }
        __syncthreads();
        each([&](float z) {
            if (z >= lo && z <= hi) {
                const float q = (hi - z) / width;   // NaN only for z == hi with width 0
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

template <int DT, bool AL>
__global__ __launch_bounds__(kFilterBlock) void filter_kernel(Params P)
{
    __shared__ FilterLds sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const int dt = DT;
    const bool target = v < P.nT;
    const void *base = vec_ptr(target ? P.target : P.draft, dt, target ? v : v - P.nT, P.V);
    const int64_t nunits = (P.V + kUnitElems - 1) / kUnitElems;

    // maximum, smallest finite logit, finite count; NaN or +inf leaves the vector
    // unfiltered (its row is reported non-finite)
    float mx = -INFINITY, mn = INFINITY;
    uint32_t nfin = 0u, bad = 0u;
    each_logit<DT, AL>(base, P.V, nunits, [&](float z) {
        if (z != z || z == INFINITY) bad = 1u;
        mx = fmaxf(mx, z);
        if (z > -INFINITY) {
            mn = fminf(mn, z);
            ++nfin;
        }
    });
    const float tmx = mx;   // this thread's maximum
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, o));
        mn = fminf(mn, __shfl_xor(mn, o));
        nfin += __shfl_xor(nfin, o);
        bad |= __shfl_xor(bad, o);
    }
    if (lane == 0) {
        sh.rf[wave][0] = mx;
        sh.rf[wave][1] = mn;
        sh.ru[wave] = nfin | (bad << 31);
    }
    __syncthreads();
    mx = -INFINITY;
    mn = INFINITY;
    nfin = 0u;
    bad = 0u;
    for (int w = 0; w < kFilterWaves; ++w) {
        mx = fmaxf(mx, sh.rf[w][0]);
        mn = fminf(mn, sh.rf[w][1]);
        nfin += sh.ru[w] & 0x7fffffffu;
        bad |= sh.ru[w] >> 31;
    }
    __syncthreads();
    if (bad || nfin == 0u) {
        if (tid == 0) P.theta[v] = -INFINITY;
        return;
    }
    const double c64 = 1.4426950408889634 / (double)vc.T;

    auto from_hbm = [&](auto &&f) { each_logit<DT, AL>(base, P.V, nunits, f); };
    auto from_cand = [&](auto &&f) {
        for (uint32_t i = tid; i < sh.ncand; i += kFilterBlock) f(sh.cand[i]);
    };
    float theta = -INFINITY;
    double S = 0.0;
    bool in_lds = false;
    // threads whose maximum is finite (each such maximum is a different logit)
    const int nmax_fin = __syncthreads_count(tmx > -INFINITY);
    if (use_k && (uint64_t)k <= nfin && k <= nmax_fin) {
        // top-k candidates: the k-th largest of the per-thread maxima is a lower bound L
        // of theta_k (those maxima are logits of the vector); the logits >= L, at
        // least k of them, usually fit in LDS and every later step runs there
        sh.tmax[tid] = tmx;
        if (tid == 0) sh.ncand = 0u;
        __syncthreads();
        auto from_tmax = [&](auto &&f) { f(sh.tmax[tid]); };
        const float L = bucket_search<false>(from_tmax, mn, mx, 0.0, (double)k, mx, c64, sh);
        from_hbm([&](float z) {
            if (z >= L) {
                const uint32_t i = atomicAdd(&sh.ncand, 1u);
                if (i < (uint32_t)kMaxCand) sh.cand[i] = z;
            }
        });
        __syncthreads();
        in_lds = sh.ncand <= (uint32_t)kMaxCand;
    }
    if (in_lds) {
        theta = bucket_search<false>(from_cand, mn, mx, 0.0, (double)k, mx, c64, sh);
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
        if (use_k && (uint64_t)k <= nfin)
            theta = bucket_search<false>(from_hbm, mn, mx, 0.0, (double)k, mx, c64, sh);
        if (use_p) {
            const float lower = theta > -INFINITY ? theta : mn;
            double s = 0.0;
            from_hbm([&](float z) {
                if (z >= lower) s += exp2_f64(((double)z - (double)mx) * c64);
            });
            const double Sk = fblock_sum(s, sh);
            theta = fmaxf(theta, bucket_search<true>(from_hbm, lower, mx, 0.0, (double)tp * Sk, mx, c64, sh));
        }
        // the filtered statistics: the maximum and the exact sum over the kept logits
        double s = 0.0;
        from_hbm([&](float z) {
            if (z >= theta) s += exp2_f64(((double)z - (double)mx) * c64);
        });
        S = fblock_sum(s, sh);
    }
    const int64_t ipv = P.geo.ipv;
    for (int64_t j = tid; j < ipv; j += kFilterBlock)
        P.parts[v * ipv + j] = j == 0 ? Partial{mx, __float_as_int(__builtin_nanf("")), S}
                                      : Partial{-INFINITY, INT32_MAX, 0.0};
    if (tid == 0) {
        P.theta[v] = theta;
        if (vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V) {
            float* zx = P.zx + (target ? 0 : P.nD) + vc.slot;
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

}  // namespace sv
