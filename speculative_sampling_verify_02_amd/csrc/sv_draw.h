// Device helpers of the draws and of the merges of per-piece records, shared by the
// kernels after the streaming pass and by the fused verification kernel: the merge of
// a vector's piece records into (max, sum), the draw weights of the residual
// max(0, p - q) and of p (rayaq.ca "Speculative decoding", section "One round", steps
// 4 and 5), and wave-level totals and prefix sums for the inverse-CDF walk.
#pragma once

#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

constexpr double kQNaN = __builtin_nan("");

// log2 of the factor that takes a record's sum to sum 2^((z - m) c) over its logits
// (0 for records of -inf or NaN logits, and for references stored as NaN: exact m c).
// A record's sum is taken against fl(ref c_hi); c_eff is the full scale.
template <int DT>
__device__ __forceinline__ double rec_shift(const Partial &q, const TempConst &tc)
{
    if (!(q.m > -INFINITY && q.m < INFINITY)) return 0.0;
    const float ref = __int_as_float(q.idx);
    if (ref != ref) return 0.0;
    return (double)(ref * tc.c_hi) - (double)q.m * tc.c_eff;
}


// Records of global vector v: items [v ipv, (v + 1) ipv).
__device__ __forceinline__ void vec_records(const Params &P, int64_t v, int64_t &i0, int64_t &i1)
{
    i0 = v * P.geo.ipv;
    i1 = i0 + P.geo.ipv - 1;
}

template <int DT>
__device__ __forceinline__ void wave_merge(const Params &P, const Partial &q0, int64_t i0, int64_t i1, bool greedy,
                                           const TempConst &tc, int lane, float &M, double &S, int32_t &idx)
{
    float m = q0.m;
    double s = greedy ? 0.0 : q0.s;
    double sh = greedy ? 0.0 : rec_shift<DT>(q0, tc);   // s 2^sh: sum 2^((z - m) c) of this lane's logits
    int32_t id = (m != m) ? INT32_MAX : q0.idx;
    for (int64_t i = i0 + 64 + lane; i <= i1; i += 64) {   // vectors of more than 64 items
        const Partial q = P.parts[i];
        if (greedy) {
            if (q.m != q.m) {
                m = q.m;
            } else if (q.m > m) {
                m = q.m;
                id = q.idx;
            } else if (q.m == m && q.idx < id) {
                id = q.idx;
            }
            continue;
        }
        s *= exp2_f64(sh);
        sh = 0.0;
        const double qs = q.s * exp2_f64(rec_shift<DT>(q, tc));
        if (q.m > m) {
            if (m != -INFINITY) s *= exp2_f64(((double)m - (double)q.m) * tc.c_eff);
            m = q.m;
        }
        s += q.m == -INFINITY ? qs : qs * exp2_f64(((double)q.m - (double)m) * tc.c_eff);
        if (q.m != q.m) m = q.m;
    }
    M = wave_umax_f32(m);
    if (greedy) {
        S = 0.0;
        idx = wave_umin_i32(m == M ? id : INT32_MAX);
    } else {
        // NaN anywhere gives M = NaN and S = NaN
        const double t = m == -INFINITY ? s : s * exp2_f64(sh + ((double)m - (double)M) * tc.c_eff);
        S = wave_usum_f64(t);
        idx = INT32_MAX;
    }
}

// Bytes of the target (or draft) logit array.
__device__ __forceinline__ uint64_t array_bytes(const Params &P, int DT, bool target)
{
    return (uint64_t)(target ? P.nT : P.nD) * (uint64_t)P.V * (DT == 0 ? 2u : 4u);
}

// A unit past the end of a vector, read as -inf logits.
template <int DT>
__device__ __forceinline__ RawUnit<DT> neg_inf_unit()
{
    RawUnit<DT> r;
    if constexpr (DT == 0) {
        r.a = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    } else {
        r.a = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        r.b = r.a;
    }
    return r;
}

template <int DT>
struct DrawConst;

// bf16 logits: fp32 weights 2^((z - m) c) / S.  The difference z - m of two bf16
// values is exact in fp32, so the maximum gets exactly 1 / S: a distribution that
// keeps one token (a top-k 1 filter) has weight exactly 1 there on both models.
template <>
struct DrawConst<0> {
    float c, mt, md, Ft, Fd, tht, thd;
    float r;       // S_t / S_d: q's weights 2^((z - m_d) c) on p's scale (residual draws)
    double Ftd;    // 1 / S_t in fp64, the scale of unit_sums
    bool residual;
    bool filt;   // a threshold applies (filtered call): logits below it drop out

    __device__ __forceinline__ void init(const RowDraw &D)
    {
        tht = D.theta_t;
        thd = D.theta_d;
        c = temp_const<0>(D.T).c_hi;
        residual = D.kind == DRAW_RESIDUAL;
        mt = D.m_t;
        Ft = (float)(1.0 / D.S_t);
        md = D.m_d;
        Fd = residual ? (float)(1.0 / D.S_d) : 0.0f;
        r = residual ? (float)(D.S_t / D.S_d) : 0.0f;
        Ftd = 1.0 / D.S_t;
        filt = tht > -INFINITY || thd > -INFINITY;
    }
    // A unit's sums of w and of p before the common factor 1 / S_t (Ftd): p's terms
    // 2^((z_t - m_t) c), w's max(0, 2^((z_t - m_t) c) - r 2^((z_d - m_d) c)) for a
    // residual draw, else p's.  Equal p and q (S_t = S_d, so r = 1) still cancel to 0.
    template <bool FILT, int RES>
    __device__ __forceinline__ void unit_sums(const float *zt, const float *zd, float &sw, float &sp) const
    {
        sw = 0.0f;
        sp = 0.0f;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const float zte = (FILT && zt[e] < tht) ? -INFINITY : zt[e];
            const float a = hw_exp2((zte - mt) * c);
            sp += a;
            if (RES) {
                const float zde = (FILT && zd[e] < thd) ? -INFINITY : zd[e];
                sw += fmaxf(0.0f, fmaf(-r, hw_exp2((zde - md) * c), a));
            }
        }
        if (!RES) sw = sp;
    }
    using W = float;
    // weights of one unit: w (residual or p) and p; FILT false: no threshold applies
    // (the comparisons skipped); RES 0 or 1 fixes the kind of draw at compile time (the
    // draft's exponentials skipped, or taken without a branch), -1 reads it from the row
    template <bool FILT = true, int RES = -1>
    __device__ __forceinline__ void weights(const float *zt, const float *zd, float *w, float *p) const
    {
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            // logits below a filter's threshold drop out
            const float zte = (FILT && zt[e] < tht) ? -INFINITY : zt[e];
            const float zde = (FILT && zd[e] < thd) ? -INFINITY : zd[e];
            const float pe = hw_exp2((zte - mt) * c) * Ft;
            float we = pe;
            if (RES == 1 || (RES < 0 && residual)) we = fmaxf(0.0f, pe - hw_exp2((zde - md) * c) * Fd);
            w[e] = we;
            p[e] = pe;
        }
    }
};

// 1 - 2^y for y <= 0.  Near 0, where 2^y is close to 1 and the difference would
// lose its relative accuracy, from the series -sum_k (y ln 2)^k / k! to degree 8
// (y > -1/2: truncation below 1e-9 relative); below, from the hardware exp2.
__device__ __forceinline__ float one_minus_exp2(float y)
{
    float s = (float)kExp2Coef[5];   // (ln 2)^8 / 8!; kExp2Coef[13 - k] = (ln 2)^k / k!
#pragma unroll
    for (int k = 7; k >= 1; --k) s = fmaf(s, y, (float)kExp2Coef[13 - k]);
    return y > -0.5f ? -y * s : 1.0f - hw_exp2(y);
}

// fp32 logits: fp32 weights from the hardware exp2, p = 2^(u c_hi + u c_lo - B) with the
// vector's normalisation in the exponent: B = m c + log2 S held as two fp32 parts
// (~2^-48 relative), so no per-vector factor is rounded to fp32.  When |fl(m c_hi)| <
// 2^20, u = z; otherwise u = z - m, which is exact for every logit whose weight is not
// 0 (it lies within a factor 2 of m), and B = log2 S.
// The residual is taken as p (1 - 2^y) with y = log2(q/p) = ((z_d - z_t) + (m_t - m_d)) c
// + log2(S_t / S_d) evaluated in fp64 (full rate on this GPU, fewer operations than
// carrying the differences in two fp32 parts): y keeps its relative accuracy where q
// is close to p (a difference p - q would keep only the absolute accuracy of p and q),
// and it is exactly log2(S_t / S_d), 0 for equal sums, wherever z_t - m_t = z_d - m_d,
// as for a distribution that keeps one token (both differences of fp32 values are
// then exact in fp64 and cancel).
template <>
struct DrawConst<1> {
    float ch, cl, ut, Bht, Blt, tht, thd;
    double c64, M64, L64;   // c, m_t - m_d (exact) and log2(S_t / S_d): the residual's y
    bool residual;
    bool filt;   // a threshold applies (filtered call): logits below it drop out

    __device__ __forceinline__ static void split(double x, float &hi, float &lo)
    {
        hi = (float)x;
        lo = (float)(x - (double)hi);
    }
    __device__ __forceinline__ void init(const RowDraw &D)
    {
        tht = D.theta_t;
        thd = D.theta_d;
        const TempConst tc = temp_const<1>(D.T);
        ch = tc.c_hi;
        cl = tc.c_lo;
        residual = D.kind == DRAW_RESIDUAL;
        filt = tht > -INFINITY || thd > -INFINITY;
        const double Lt = log2(D.S_t);
        double B = Lt;
        ut = D.m_t;
        if (fabsf(D.m_t * tc.c_hi) < kFastRef) {
            ut = 0.0f;
            B += (double)D.m_t * tc.c_eff;
        }
        split(B, Bht, Blt);
        c64 = tc.c_eff;
        M64 = residual ? (double)D.m_t - (double)D.m_d : 0.0;   // exact: both are fp32
        L64 = residual ? Lt - log2(D.S_d) : 0.0;
    }
    using W = float;
    // FILT false: no threshold applies (the comparisons skipped); RES 0 or 1 fixes the
    // kind of draw at compile time, -1 reads it from the row
    template <bool FILT = true, int RES = -1>
    __device__ __forceinline__ void weights(const float *zt, const float *zd, float *w, float *p) const
    {
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const float zte = (FILT && zt[e] < tht) ? -INFINITY : zt[e];
            const float xt = zte - ut;
            const float pe = hw_exp2(fmaf(xt, cl, fmaf(xt, ch, -Bht)) - Blt);
            float we = pe;
            if (RES == 1 || (RES < 0 && residual)) {
                const float zde = (FILT && zd[e] < thd) ? -INFINITY : zd[e];
                const float y = (float)fma(((double)zde - (double)zte) + M64, c64, L64);
                // without a branch: q = 0 gives y = -inf and keeps all of p (1 - 2^-inf
                // = 1); y >= 0 (q >= p) and NaN (p = q = 0) become y = 0 (minNum) and
                // keep nothing
                we = pe * one_minus_exp2(fminf(y, 0.0f));
            }
            w[e] = we;
            p[e] = pe;
        }
    }
};

// logits per draw piece (two halves of the streaming pass) and tiles per piece
template <int DT> constexpr int kPieceTiles = (int)(2 * kItemElems / kTileElems);

// Sum of p over piece q of a vector whose maximum is m and sum 2^((z - m) c) is S.
template <int DT>
__device__ __forceinline__ double piece_weight(const Partial &q, const TempConst &tc, float m, double S)
{
    if (!(q.m > -INFINITY)) return 0.0;
    return q.s * exp2_f64(rec_shift<DT>(q, tc) + ((double)q.m - (double)m) * tc.c_eff) / S;
}

// The bonus draw's piece from the pieces' p sums (lane j holds piece j): the first
// piece where the running sum exceeds t = u W, else the last one with weight.
template <int DT>
__device__ __forceinline__ void bonus_piece(const Partial &q, const TempConst &tc, float m, double S, float u,
                                            int lane, int32_t &piece, double &before, double &W)
{
    const double w = (m == m && S > 0.0) ? piece_weight<DT>(q, tc, m, S) : 0.0;
    const double incl = wave_inclusive_sum(w, lane);
    W = __shfl(incl, 63);
    const double t = (double)u * W;
    const unsigned long long hit = __ballot(incl > t && w > 0.0);
    const unsigned long long pos = __ballot(w > 0.0);
    const int l = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : -1);
    piece = l;
    before = l >= 0 ? __shfl(incl - w, l) : 0.0;
}

// Totals over the 64 lanes of N per-lane values (N a power of two, at most 64), in
// every lane: a butterfly where each exchange also halves the values a lane carries
// (log2 N steps leave lane l the partial total of value bitrev(l mod N) over its
// group of N lanes), then the groups are added, and the totals read back per value.
template <int N>
__device__ __forceinline__ void wave_totals(double (&v)[N], int lane)
{
    constexpr int LOGN = N == 1 ? 0 : N == 2 ? 1 : N == 4 ? 2 : N == 8 ? 3 : N == 16 ? 4 : N == 32 ? 5 : 6;
    static_assert((1 << LOGN) == N, "N must be a power of two up to 64");
    double x[N];
#pragma unroll
    for (int k = 0; k < N; ++k) x[k] = v[k];
#pragma unroll
    for (int st = 0; st < LOGN; ++st) {
        const int half = N >> (st + 1);
        const bool up = (lane >> st) & 1;
#pragma unroll
        for (int k = 0; k < half; ++k) {
            const double send = up ? x[k] : x[k + half];
            const double keep = up ? x[k + half] : x[k];
            x[k] = keep + __shfl_xor(send, 1 << st);
        }
    }
    double t = x[0];
#pragma unroll
    for (int m = N; m < 64; m <<= 1) t += __shfl_xor(t, m);
#pragma unroll
    for (int k = 0; k < N; ++k) {
        int r = 0;   // the lane holding value k: k with its LOGN bits reversed
#pragma unroll
        for (int bit = 0; bit < LOGN; ++bit) r |= ((k >> bit) & 1) << (LOGN - 1 - bit);
        v[k] = readlane_f64(t, r);
    }
}

}  // namespace sv
