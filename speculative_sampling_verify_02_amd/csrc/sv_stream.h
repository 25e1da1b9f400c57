// Device helpers of the streaming pass over logit vectors, shared by the kernels that
// read every logit once (the statistics pass, the early-exit steps, and the fused
// verification kernel): half-piece loads, their reduction to per-lane sums or first
// argmax, and the per-piece record.
//
// bf16 logits are summed in fp32 (exp2 on the hardware unit, the exponent from one
// fma) and added across lanes in fp64.  fp32 logits are summed term by term in fp64
// (a table-driven exp2): the residual mass of a draft close to the target depends on
// the ratio of the two sums to ~1e-9 relative, below what an fp32 exp can give.
#pragma once

#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

// ===========================================================================
// streaming pass
// ===========================================================================

// One half-piece as this lane holds it: load k covers bytes [1024 k + 16 l, +16) of
// the half.  Rows that do not start 16-byte aligned are loaded from the aligned
// address below the half's start: sb is the offset of the half's first byte there,
// and e the aligned 16 bytes after the last load's (for lane 63 of that load).
template <int DT>
struct ItemRaw {
    uint4 d[kItemLoads<DT>];
    uint4 e;
    uint32_t sb;
};

// logits per 16-byte load
template <int DT> constexpr int kE = DT == 0 ? 8 : 4;

// Logits of piece j of vector v in half h: [j 2 ie + h ie, +n), n in [0, ie].
__device__ __forceinline__ int32_t half_len(const Params &P, int64_t j, int h)
{
    const int64_t e0 = (2 * j + h) * P.geo.ie;
    const int64_t n = P.V - e0;
    return (int32_t)(n < 0 ? 0 : (n < P.geo.ie ? n : P.geo.ie));
}

// Issue the loads of half h of piece j of vector v.  Aligned rows: offsets past the
// end of the vector are clamped to its last 16 bytes (those logits are masked when
// the half is reduced).  Other rows: aligned blocks from below the half's start,
// moved into place by realign.  An empty half, or live = false (no piece left), reads
// an empty window at the start of the vector (nothing to read, nothing used), which
// keeps every load of the pipeline unconditional.
template <int DT, bool AL>
__device__ __forceinline__ void half_begin(const Params &P, int64_t v, int64_t j, int h, bool live, ItemRaw<DT> &r,
                                           int lane)
{
    constexpr int64_t esz = DT == 0 ? 2 : 4;
    if (!live) v = j = 0;
    const int64_t n = live ? half_len(P, j, h) : 0;
    const bool target = v < P.nT;
    const int64_t row = target ? v : v - P.nT;
    const int64_t e0 = n > 0 ? (2 * j + h) * P.geo.ie : 0;
    const char *base = static_cast<const char *>(target ? P.target : P.draft) + (row * P.V + e0) * esz;
    if constexpr (AL) {
        const uint32_t nbytes = (uint32_t)(n * esz);   // a multiple of 16
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, (int)nbytes, kBufferWord3);
        const uint32_t last = nbytes > 16u ? nbytes - 16u : 0u;
#pragma unroll
        for (int k = 0; k < kItemLoads<DT>; ++k) {
            uint32_t off = (uint32_t)k * 1024u + (uint32_t)lane * 16u;
            off = off < last ? off : last;
            r.d[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, kLoadNT));
        }
    } else {
        // aligned 16-byte loads from the aligned address at or below the half's start,
        // each clamped to the last aligned 16 bytes that hold a byte of the array (a
        // 16-byte block holding a valid byte lies in a mapped page; what the clamp
        // replaces lies past the array, hence past the row, and is masked); the bytes
        // are moved into place by realign before the half is reduced
        const char *arr = static_cast<const char *>(target ? P.target : P.draft);
        const uint64_t arr_bytes = (uint64_t)(target ? P.nT : P.nD) * (uint64_t)P.V * (uint64_t)esz;
        const uint64_t a = reinterpret_cast<uint64_t>(base);
        const uint64_t a0 = a & ~(uint64_t)15;
        const uint64_t last = (reinterpret_cast<uint64_t>(arr) + arr_bytes - 1) & ~(uint64_t)15;
        r.sb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(a - a0));
#pragma unroll
        for (int k = 0; k < kItemLoads<DT>; ++k) {
            uint64_t q = a0 + (uint64_t)(k * 64 + lane) * 16u;
            q = q < last ? q : last;
            r.d[k] = load_nt16(reinterpret_cast<const void *>(q));
        }
        uint64_t qe = a0 + (uint64_t)kItemLoads<DT> * 1024u;
        qe = qe < last ? qe : last;
        r.e = load_nt16(reinterpret_cast<const void *>(qe));
    }
}

// Moves an unaligned half's bytes into the aligned layout: lane l of load k takes the
// 16 bytes at offset sb of its own aligned block and the next one (lane l + 1's, or
// for lane 63 lane 0's of load k + 1, or e after the last load).
template <int DT, int Q>
__device__ __forceinline__ void realign_q(ItemRaw<DT> &r, int lane, uint32_t rb)
{
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        uint4 nx = make_uint4(wave_next_lane(r.d[k].x), wave_next_lane(r.d[k].y), wave_next_lane(r.d[k].z),
                              wave_next_lane(r.d[k].w));
        const uint4 l0 = k + 1 < kItemLoads<DT>
            ? make_uint4((uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].x, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].y, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].z, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].w, 0))
            : r.e;
        if (lane == 63) nx = l0;
        r.d[k] = funnel16<Q>(r.d[k], nx, rb);
    }
}

template <int DT>
__device__ __forceinline__ void realign(ItemRaw<DT> &r, int lane)
{
    const uint32_t rb = r.sb & 3u;
    switch (r.sb >> 2) {
    case 0: if (rb != 0) realign_q<DT, 0>(r, lane, rb); break;
    case 1: realign_q<DT, 1>(r, lane, rb); break;
    case 2: realign_q<DT, 2>(r, lane, rb); break;
    default: realign_q<DT, 3>(r, lane, rb); break;
    }
}

// Logits at half offsets n and beyond become -inf (the short end of a vector).  With
// AL the rows hold whole 16-byte loads, so the test is per load.
template <int DT, bool AL>
__device__ __forceinline__ void mask_tail(ItemRaw<DT> &r, int lane, int n)
{
    constexpr int E = kE<DT>;
    constexpr uint32_t kNinf = DT == 0 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        if constexpr (AL) {
            if (k * 64 * E + lane * E >= n) r.d[k] = make_uint4(kNinf, kNinf, kNinf, kNinf);
        } else {
            uint32_t w[4] = {r.d[k].x, r.d[k].y, r.d[k].z, r.d[k].w};
#pragma unroll
            for (int t = 0; t < E; ++t) {
                if (k * 64 * E + lane * E + t < n) continue;
                if constexpr (DT == 0) w[t / 2] = (t & 1) ? ((w[t / 2] & 0xffffu) | 0xff800000u) : ((w[t / 2] & 0xffff0000u) | 0xff80u);
                else w[t] = 0xff800000u;
            }
            r.d[k] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// bf16 pairs to fp32 by byte permutes (two operand orders): other ways of unpacking,
// so that a pass that re-reads the registers recomputes the values instead of keeping
// an earlier pass's (or another branch's) values live
template <int FORM>
__device__ __forceinline__ float bf16_lo_f(uint32_t w)
{
    return __uint_as_float(FORM == 1 ? __builtin_amdgcn_perm(0u, w, 0x01000c0cu) : __builtin_amdgcn_perm(w, 0u, 0x05040c0cu));
}
template <int FORM>
__device__ __forceinline__ float bf16_hi_f(uint32_t w)
{
    return __uint_as_float(FORM == 1 ? __builtin_amdgcn_perm(0u, w, 0x03020c0cu) : __builtin_amdgcn_perm(w, 0u, 0x07060c0cu));
}

// The logits of load k on this lane (FORM picks the bf16 unpacking: 0 shifts and
// masks, 1 and 2 byte permutes).
template <int DT, int FORM = 0>
__device__ __forceinline__ void lane_vals(const ItemRaw<DT> &r, int k, float *x)
{
    const uint4 w = r.d[k];
    if constexpr (DT == 0 && FORM != 0) {
        x[0] = bf16_lo_f<FORM>(w.x); x[1] = bf16_hi_f<FORM>(w.x);
        x[2] = bf16_lo_f<FORM>(w.y); x[3] = bf16_hi_f<FORM>(w.y);
        x[4] = bf16_lo_f<FORM>(w.z); x[5] = bf16_hi_f<FORM>(w.z);
        x[6] = bf16_lo_f<FORM>(w.w); x[7] = bf16_hi_f<FORM>(w.w);
    } else if constexpr (DT == 0) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
        x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    } else {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
}

template <int DT>
__device__ __forceinline__ float lane_max(const ItemRaw<DT> &r)
{
    constexpr int E = kE<DT>;
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[E];
        lane_vals<DT>(r, k, x);
#pragma unroll
        for (int t = 0; t < E; ++t) m = nmax(m, x[t]);
    }
    return m;
}

__device__ __forceinline__ float wave_usum_f32(float v)
{
    v += dpp_f32<0x121>(v);
    v += dpp_f32<0x122>(v);
    v += dpp_f32<0x124>(v);
    v += dpp_f32<0x128>(v);
    return v;
}

// fp64 total of a wave of fp32 lane values (fp32 within rows of 16 lanes)
__device__ __forceinline__ double wave_total(float v)
{
    v = wave_usum_f32(v);
    return ((double)readlane_f32(v, 0) + (double)readlane_f32(v, 16)) +
           ((double)readlane_f32(v, 32) + (double)readlane_f32(v, 48));
}

// 2^d for a double d in fp32: the integer part exactly, the fraction on the hardware unit
__device__ __forceinline__ float exp2_split(double d)
{
    const double n = rint(d);
    return ldexpf(hw_exp2((float)(d - n)), (int)n);
}

// ---------------------------------------------------------------------------
// bf16 sampling piece.  Every lane sums 2^(z c - E) over its logits against its
// own reference E: E = B = fl(R c) for a reference logit R (E = B + fma(R, c, -B),
// the exact R c, when |B| >= 2^30, where the rounding of B would matter).  R starts
// as the largest logit of the lane's first load; when a lane's sum over a half
// overflows (a logit far above R) the half is summed again, from registers, against
// the lane's maximum.  The epilogue brings the lanes to the piece maximum M.
// ---------------------------------------------------------------------------
struct LaneSum {
    float m;      // maximum so far (NaN-propagating)
    float s;      // sum 2^(z c - E) so far (0 while m = -inf)
    double s64;   // fp32 logits: the same sum in fp64
    float Bhi;    // fl(R c)
    float Blo;    // R c - Bhi (used when huge)
    double E;     // the reference of s
    bool huge;    // wave-uniform: the two-part reference is in use
};

__device__ __forceinline__ void set_ref(LaneSum &a, float R, float c)
{
    a.Bhi = R * c;
    a.Blo = fmaf(R, c, -a.Bhi);
    a.huge = __any(!(fabsf(a.Bhi) < 0x1p30f));
    a.E = a.huge ? (double)a.Bhi + (double)a.Blo : (double)a.Bhi;
}

// add one bf16 half (first: the piece's first half, which sets the references); the
// term of logit x is 2^(x c - Bhi), one fma and the hardware exp2
__device__ __forceinline__ void sample_half(const ItemRaw<0> &r, float c, LaneSum &a, bool first)
{
    constexpr int DT = 0;
    constexpr int E = kE<DT>;
    if (first) {
        float x[E];
        lane_vals<DT>(r, 0, x);
        float R = x[0];
#pragma unroll
        for (int t = 1; t < E; ++t) R = nmax(R, x[t]);
        a.m = -INFINITY;
        a.s = 0.0f;
        set_ref(a, R, c);
    }
    const float m_prev = a.m, s_prev = a.s;
    const double E_prev = a.E;
    float acc[kItemLoads<DT>];
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[E];
        lane_vals<DT, 1>(r, k, x);
#pragma unroll
        for (int t = 0; t < E; ++t) a.m = nmax(a.m, x[t]);
#pragma unroll
        for (int t = 0; t < E; ++t) x[t] = hw_exp2(fmaf(x[t], c, -a.Bhi));
#pragma unroll
        for (int w = 1; w < E; w <<= 1)
#pragma unroll
            for (int t = 0; t + w < E; t += 2 * w) x[t] += x[t + w];
        acc[k] = x[0];
    }
#pragma unroll
    for (int w = 1; w < kItemLoads<DT>; w <<= 1)
#pragma unroll
        for (int k = 0; k + w < kItemLoads<DT>; k += 2 * w) acc[k] += acc[k + w];
    // a lane whose logits are finite but whose sum is not, or a two-part reference: the
    // references move to the lanes' maxima, the earlier sum is rescaled, and the half is
    // summed again (from registers) with the two-part reference when needed
    const bool over = !(acc[0] <= 3.402823466e38f) && fabsf(a.m) <= 3.402823466e38f;
    if (__any(over) || a.huge) {
        const float R = fabsf(a.m) <= 3.402823466e38f ? a.m : 0.0f;
        set_ref(a, R, c);
        a.s = m_prev == -INFINITY ? 0.0f : s_prev * (float)exp2_f64(E_prev - a.E);
        const float Blo = a.huge ? a.Blo : 0.0f;
        float acc2[kItemLoads<DT>];
#pragma unroll
        for (int k = 0; k < kItemLoads<DT>; ++k) {
            float x[E];
            lane_vals<DT, 2>(r, k, x);
#pragma unroll
            for (int t = 0; t < E; ++t) x[t] = hw_exp2(fmaf(x[t], c, -a.Bhi) - Blo);
#pragma unroll
            for (int w = 1; w < E; w <<= 1)
#pragma unroll
                for (int t = 0; t + w < E; t += 2 * w) x[t] += x[t + w];
            acc2[k] = x[0];
        }
#pragma unroll
        for (int w = 1; w < kItemLoads<DT>; w <<= 1)
#pragma unroll
            for (int k = 0; k + w < kItemLoads<DT>; k += 2 * w) acc2[k] += acc2[k + w];
        acc[0] = acc2[0];
    }
    a.s += acc[0];
    if (a.m == -INFINITY) a.s = 0.0f;
}

// 2^(a/L) in fp64 from a table of the L = 256 values 2^(j/L) in LDS (exp2_tab_read,
// then exp2_tab_add): a = k + r with k = rint(a), so |r| <= 1/2 and
// 2^(a/L) = 2^floor(k/L) 2^((k mod L)/L) 2^(r/L), with 2^(r/L) from its Taylor series
// in r ln 2 / L to degree 2 (truncation below (ln 2 / 512)^3 / 6 = 4.2e-10 relative).
// The power 2^floor(k/L) scales the table entry (ldexp, exact): the caller keeps
// a >= -1000 L (2^-1000, a term that cannot register next to the maximum's 1), so the
// scaled entry stays normal.  Entry j of the lane's copy is at col[j << sh] (sh = 6:
// one column per lane, which no two lanes of a wave share, so the reads meet no bank
// conflicts; sh = 0: a single shared copy).  With 64 columns the table takes 128 KB
// of LDS, which the streaming kernel's one workgroup per CU can hold.
constexpr int kTabBits = 8;
constexpr int kTabLen = 1 << kTabBits;

struct Exp2Tab {
    const double *col;
    int sh;
};

// (ln 2 / L)^j / j!  (kExp2Coef[13 - j] = (ln 2)^j / j!, scaled by L^-j exactly)
constexpr double kTabC1 = kExp2Coef[12] / kTabLen;
constexpr double kTabC2 = kExp2Coef[11] / kTabLen / kTabLen;

// The two halves of exp2_tab, so that a caller can issue the table reads of several
// terms before it waits for the first: the rounding and the read, then the series.
struct TabTerm {
    double r;   // a - rint(a)
    double T;   // 2^((k mod L)/L)
    int ki;     // rint(a)
};

__host__ __device__ __forceinline__ TabTerm exp2_tab_read(double a, const Exp2Tab &t)
{
    const double k = rint(a);
    TabTerm u;
    u.r = a - k;   // exact
    u.ki = (int)k;
    u.T = t.col[(u.ki & (kTabLen - 1)) << t.sh];
    return u;
}

// s + 2^(a/L): the table entry scaled by 2^floor(k/L) (ldexp: a term down to 2^-1000
// stays exact), times the series, added to s in one fma.
__host__ __device__ __forceinline__ double exp2_tab_add(const TabTerm &u, double s)
{
    const double q = fma(fma(kTabC2, u.r, kTabC1), u.r, 1.0);
    return fma(ldexp(u.T, u.ki >> kTabBits), q, s);
}

// Entry j of the table, 2^(j/L).
__host__ __device__ __forceinline__ double exp2_tab_entry(int j)
{
    return exp2_f64((double)j * (1.0 / kTabLen));
}

// Fill a table of 2^(j/L) for exp2_tab_read: kTabLen entries, each repeated `copies`
// times (64: one column per lane; 1: a single copy), by a workgroup of NT threads.  The
// caller synchronises after it.
template <int NT>
__device__ __forceinline__ void fill_exp2_tab(double *tab, int copies)
{
    for (int i = threadIdx.x; i < kTabLen * copies; i += NT) tab[i] = exp2_tab_entry(i / copies);
}

// fp32 logits: the sums feed log2(S_t / S_d), which the residual mass of a draft close
// to the target needs to ~1e-9 relative, so every term is an fp64 2^(x c - E): the
// exponent from one fp64 fma (c the full scale), the power from the table.  The half's
// lane maximum comes first and the reference follows the running lane maximum (the
// sum so far rescaled), so every exponent is <= 0 up to rounding.
__device__ __forceinline__ void sample_half_f32(const ItemRaw<1> &r, double c_eff, LaneSum &a, bool first,
                                                const Exp2Tab &tab)
{
    constexpr int DT = 1;
    float mh = -INFINITY;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[4];
        lane_vals<1>(r, k, x);
#pragma unroll
        for (int t = 0; t < 4; ++t) mh = nmax(mh, x[t]);
    }
    const float mprev = first ? -INFINITY : a.m;
    const float mnew = nmax(mprev, mh);
    // the reference is R c with the full scale, in fp64 (against R c_hi alone the term
    // of R itself would be 2^(R c_lo), which overflows once R c passes ~2^33)
    if (first) {
        a.s64 = 0.0;
        a.E = (double)(fabsf(mnew) <= 3.402823466e38f ? mnew : 0.0f) * c_eff;
    } else if (fabsf(mnew) <= 3.402823466e38f && mnew > mprev) {
        const double E_old = a.E;
        a.E = (double)mnew * c_eff;
        a.s64 = mprev == -INFINITY ? 0.0 : a.s64 * exp2_f64(E_old - a.E);
    }
    a.m = mnew;
    if (!(fabsf(mnew) <= 3.402823466e38f)) return;   // -inf so far (nothing to add), or NaN / +inf
    // exponents scaled by L (exact) and kept >= -1000 L (-inf logits included)
    const double cs = (double)kTabLen * c_eff, Es = (double)kTabLen * a.E;
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[4];
        lane_vals<1, 1>(r, k, x);
        TabTerm u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = exp2_tab_read(fmax(fma((double)x[t], cs, -Es), -1000.0 * kTabLen), tab);
#pragma unroll
        for (int t = 0; t < 4; ++t) s = exp2_tab_add(u[t], s);
    }
    a.s64 += s;
}

// The piece's record from the lane sums: m = M, s = sum 2^(z c' - E_M) (c' = c + c_lo,
// the scale) with E_M = fl(M c) (ref = M, in idx) or, when |fl(M c)| >= 2^30, the
// exact M c' (ref = NaN).
template <int DT>
__device__ __forceinline__ Partial sample_record(const LaneSum &a, float c, float c_lo)
{
    const float M = wave_umax_f32(a.m);
    Partial p{M, 0, 0.0};
    if (M == -INFINITY) return p;
    if (!(fabsf(M) <= 3.402823466e38f)) {   // a NaN or +inf logit
        p.idx = __float_as_int(__builtin_nanf(""));
        p.s = (double)__builtin_nanf("");
        return p;
    }
    const float BM = M * c;
    const bool exact = !(fabsf(BM) < 0x1p30f);
    const double EM = exact ? (double)M * (double)c + (double)M * (double)c_lo : (double)BM;
    p.idx = __float_as_int(exact ? __builtin_nanf("") : M);
    if constexpr (DT == 0) {
        const float t = a.m == -INFINITY ? 0.0f : a.s * exp2_split(a.E - EM);
        p.s = wave_total(t);
    } else {
        const double t = a.m == -INFINITY ? 0.0 : a.s64 * exp2_f64(a.E - EM);
        p.s = wave_usum_f64(t);
    }
    return p;
}

// ---------------------------------------------------------------------------
// greedy piece: first index of the maximum (per lane, then across the wave)
// ---------------------------------------------------------------------------
struct LaneArg {
    float best;
    int32_t idx;   // piece offset
    bool nan;
};

template <int DT>
__device__ __forceinline__ void argmax_half(const ItemRaw<DT> &r, int lane, int base, LaneArg &a)
{
    constexpr int E = kE<DT>;
    // per load maximum, then the first load holding the half's lane maximum (strictly
    // greater wins, so the earliest load keeps ties)
    float mh = -INFINITY;
    int kb = 0;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[E];
        lane_vals<DT>(r, k, x);
        float lm = x[0];
#pragma unroll
        for (int t = 1; t < E; ++t) lm = nmax(lm, x[t]);
        nan |= lm != lm;
        if (lm > mh) {
            mh = lm;
            kb = k;
        }
    }
    a.nan |= nan;
    // the first logit of that load equal to it
    uint4 w = r.d[0];
#pragma unroll
    for (int k = 1; k < kItemLoads<DT>; ++k)
        if (k == kb) w = r.d[k];
    ItemRaw<DT> one;
    one.d[0] = w;
    float x[E];
    lane_vals<DT, 1>(one, 0, x);
    int t0 = E - 1;
#pragma unroll
    for (int t = E - 2; t >= 0; --t)
        if (x[t] == mh) t0 = t;
    if (mh > a.best) {
        a.best = mh;
        a.idx = base + kb * 64 * E + lane * E + t0;
    }
}

__device__ __forceinline__ Partial argmax_record(const LaneArg &a)
{
    const float M = wave_umax_f32(a.nan ? __builtin_nanf("") : a.best);
    return Partial{M, wave_umin_i32(a.best == M ? a.idx : INT32_MAX), 0.0};
}


// ---------------------------------------------------------------------------
// the logit at the position's draft token
// ---------------------------------------------------------------------------
// The logit at half offset o (on the lane that loaded it): the raw word is picked
// with constant indices (the half stays in registers) and unpacked alone.
template <int DT>
__device__ __forceinline__ float half_value(const ItemRaw<DT> &r, int lane, int o)
{
    constexpr int E = kE<DT>;
    uint32_t wsel = 0u;
    bool hi = false;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        const uint32_t w[4] = {r.d[k].x, r.d[k].y, r.d[k].z, r.d[k].w};
#pragma unroll
        for (int t = 0; t < E; ++t) {
            if (k * 64 * E + lane * E + t == o) {
                wsel = w[DT == 0 ? t / 2 : t];
                hi = (t & 1) != 0;
            }
        }
    }
    if constexpr (DT == 0) return hi ? bf16_hi(wsel) : bf16_lo(wsel);
    else return __uint_as_float(wsel);
}

// What one piece's reduction carries between its two halves.
template <int DT>
struct PieceAcc {
    LaneSum ls;
    LaneArg la;
    float um = -INFINITY;   // UM: the maximum of the 64-logit unit this lane stores
};

// Filtered calls cut every vector into units of 64 consecutive logits: one load of G
// neighbouring lanes (G E = 64).  Each lane's load maxima are reduced over its group
// (butterfly within rows of 16 lanes), and lane l = G g + r keeps the maximum of load
// r of the piece (half r / loads, load r % loads) for group g: unit r E + g of the
// piece, logits [64 (r E + g), +64).
template <int DT>
__device__ __forceinline__ void unit_max_half(const float *lmk, int h, int lane, float &um)
{
    constexpr int E = kE<DT>, G = 64 / E, NL = kItemLoads<DT>;
    const int r = lane & (G - 1);
#pragma unroll
    for (int k = 0; k < NL; ++k) {
        float v = lmk[k];
        v = nmax(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
        v = nmax(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
        v = nmax(v, dpp_f32<0x141>(v));   // row_half_mirror: 8 lanes
        if constexpr (G == 16) v = nmax(v, dpp_f32<0x140>(v));   // row_mirror: 16 lanes
        if (r == h * NL + k) um = v;
    }
}

// The maximum of each load's logits (lmk), and the lane maximum m updated with them.
template <int DT>
__device__ __forceinline__ void max_half(const ItemRaw<DT> &r, float *lmk, float &m)
{
    constexpr int E = kE<DT>;
#pragma unroll
    for (int k = 0; k < kItemLoads<DT>; ++k) {
        float x[E];
        lane_vals<DT>(r, k, x);
        float lm = x[0];
#pragma unroll
        for (int t = 1; t < E; ++t) lm = nmax(lm, x[t]);
        lmk[k] = lm;
        m = nmax(m, lm);
    }
}

// UM with filt (a row of a filtered call that filters): the vector's sums are not
// needed, since the threshold search replaces its record by the exact sum over the
// kept logits; the half gives only the maxima (the lane's, and its unit's).
template <int DT, bool AL, bool UM = false>
__device__ __forceinline__ void piece_half(const Params &P, const VecCtx &vc, int32_t rm, const TempConst &tc,
                                           int64_t j, int h, int n, ItemRaw<DT> &r, PieceAcc<DT> &acc, int lane,
                                           const Exp2Tab &tab, bool filt = false)
{
    constexpr int E = kE<DT>;
    if constexpr (!AL) realign(r, lane);
    if (n != (int)P.geo.ie) mask_tail<DT, AL>(r, lane, n);
    if (rm == ROW_SAMPLE) {
        if (UM && filt) {
            float lmk[kItemLoads<DT>];
            if (h == 0) {
                acc.ls.m = -INFINITY;
                acc.um = -INFINITY;   // (a piece without a second half: its units are past the end)
            }
            max_half<DT>(r, lmk, acc.ls.m);
            unit_max_half<DT>(lmk, h, lane, acc.um);
        } else {
            if constexpr (DT == 0) sample_half(r, tc.c_hi, acc.ls, h == 0);
            else sample_half_f32(r, tc.c_eff, acc.ls, h == 0, tab);
        }
        // the logit at the position's draft token, if this half holds it
        if (vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V) {
            const int64_t o = (int64_t)vc.x - (2 * j + h) * P.geo.ie;
            if (o >= 0 && o < n) {
                const float z = half_value<DT>(r, lane, (int)o);
                if (lane == (int)((o % (64 * E)) / E)) P.zx[(vc.target ? 0 : P.nD) + vc.slot] = z;
            }
        }
    } else if (rm == ROW_BAD_TEMP) {
        // an unusable temperature: only the maximum (NaN-propagating) of every vector is
        // kept, which is enough to tell a position's logits non-finite
        if (h == 0) acc.la = LaneArg{-INFINITY, INT32_MAX, false};
        argmax_half<DT>(r, lane, h * (int)P.geo.ie, acc.la);
    } else if (rm == ROW_GREEDY && vc.target) {
        if (h == 0) acc.la = LaneArg{-INFINITY, INT32_MAX, false};
        argmax_half<DT>(r, lane, h * (int)P.geo.ie, acc.la);
    }
}

// The record of piece j of a vector (wave-uniform): (max, sum) for sampling rows, the
// first argmax for greedy rows' target vectors, the maximum for rows whose temperature
// is unusable.
template <int DT>
__device__ __forceinline__ Partial piece_record(const Params &P, const VecCtx &vc, int32_t rm, const TempConst &tc,
                                                int64_t j, const PieceAcc<DT> &acc, bool filt = false)
{
    Partial rec{-INFINITY, INT32_MAX, 0.0};
    if (rm == ROW_SAMPLE && filt) {
        // the maximum alone (its sum comes from the threshold search); a NaN or +inf
        // logit makes the record non-finite as in sample_record
        const float M = wave_umax_f32(acc.ls.m);
        rec = Partial{M, 0, 0.0};
        if (M == INFINITY || M != M) rec = Partial{M, __float_as_int(__builtin_nanf("")), (double)__builtin_nanf("")};
    } else if (rm == ROW_SAMPLE) {
        rec = sample_record<DT>(acc.ls, tc.c_hi, tc.c_lo);
    } else if ((rm == ROW_GREEDY && vc.target) || rm == ROW_BAD_TEMP) {
        rec = argmax_record(acc.la);
        if (rec.idx != INT32_MAX) rec.idx += (int32_t)(j * 2 * P.geo.ie);
    }
    return rec;
}

// UM (filtered calls): a sampling row that filters also stores the maximum of each of
// the piece's 64 units as a 16-bit key (unit_max_half), from which the threshold
// search bounds the top-k.
// lds_keys, lds_rec: where the piece's 64 keys and its record go instead of memory
// (the workgroup writes them out later), or null.
template <int DT, bool UM = false>
__device__ __forceinline__ void piece_finish(const Params &P, const VecCtx &vc, int32_t rm, const TempConst &tc,
                                             int64_t v, int64_t j, PieceAcc<DT> &acc, bool filt = false,
                                             uint16_t *lds_keys = nullptr, Partial *lds_rec = nullptr)
{
    const Partial rec = piece_record<DT>(P, vc, rm, tc, j, acc, UM && filt);
    const int lane = threadIdx.x & 63;
    if constexpr (UM) {
        constexpr int E = kE<DT>, G = 64 / E;
        if (rm == ROW_SAMPLE && filt) {
            const uint16_t key = unit_key(acc.um);
            const int u = (lane % G) * E + lane / G;
            if (lds_keys) lds_keys[u] = key;
            else P.umax[(v * P.geo.ipv + j) * kPieceUnits + u] = key;
        }
    }
    if (lane == 0) {
        if (lds_rec) *lds_rec = rec;
        else P.parts[v * P.geo.ipv + j] = rec;
    }
}

}  // namespace sv
