// The streaming pass of the speculative-sampling verification step for gfx950.
//
// Every logit of every target and draft vector is read exactly once.  The vectors
// are cut into pieces of two 8 KB halves; one workgroup per CU owns a contiguous
// range of pieces and its waves take them in order from a counter in LDS, each half
// as eight 16-byte loads per lane with the next half's loads in flight while one is
// reduced.  Per piece a wave writes one record: the maximum and the sum of
// 2^((z - m) c), c = log2(e)/T, over the piece (sampling rows) or the first argmax
// (greedy rows).  The temperature softmax these summarize is the softened output of
// brunomaga.github.io "inference-distillation-speculative-decoding", section
// "Knowledge distillation", with one T for both models (rayaq.ca "Speculative
// decoding", section "Why the output is exactly the target's").  The wave also keeps
// the logit at each position's draft token when it passes through its registers.
//
// bf16 logits are summed in fp32 (exp2 on the hardware unit, the exponent from one
// fma) and added across lanes in fp64.  fp32 logits are summed term by term in fp64
// (a table-driven exp2): the residual mass of a draft close to the target depends on
// the ratio of the two sums to ~1e-9 relative, below what an fp32 exp can give.
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
struct ItemRaw {
    uint4 d[kItemLoads];
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
__device__ __forceinline__ void half_begin(const Params &P, int64_t v, int64_t j, int h, bool live, ItemRaw &r,
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
        for (int k = 0; k < kItemLoads; ++k) {
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
        for (int k = 0; k < kItemLoads; ++k) {
            uint64_t q = a0 + (uint64_t)(k * 64 + lane) * 16u;
            q = q < last ? q : last;
            r.d[k] = load_nt16(reinterpret_cast<const void *>(q));
        }
        uint64_t qe = a0 + (uint64_t)kItemLoads * 1024u;
        qe = qe < last ? qe : last;
        r.e = load_nt16(reinterpret_cast<const void *>(qe));
    }
}

// Moves an unaligned half's bytes into the aligned layout: lane l of load k takes the
// 16 bytes at offset sb of its own aligned block and the next one (lane l + 1's, or
// for lane 63 lane 0's of load k + 1, or e after the last load).
template <int Q>
__device__ __forceinline__ void realign_q(ItemRaw &r, int lane, uint32_t rb)
{
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
        uint4 nx = make_uint4(wave_next_lane(r.d[k].x), wave_next_lane(r.d[k].y), wave_next_lane(r.d[k].z),
                              wave_next_lane(r.d[k].w));
        const uint4 l0 = k + 1 < kItemLoads
            ? make_uint4((uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].x, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].y, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].z, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)r.d[k + 1].w, 0))
            : r.e;
        if (lane == 63) nx = l0;
        r.d[k] = funnel16<Q>(r.d[k], nx, rb);
    }
}

__device__ __forceinline__ void realign(ItemRaw &r, int lane)
{
    const uint32_t rb = r.sb & 3u;
    switch (r.sb >> 2) {
    case 0: if (rb != 0) realign_q<0>(r, lane, rb); break;
    case 1: realign_q<1>(r, lane, rb); break;
    case 2: realign_q<2>(r, lane, rb); break;
    default: realign_q<3>(r, lane, rb); break;
    }
}

// Logits at half offsets n and beyond become -inf (the short end of a vector).  With
// AL the rows hold whole 16-byte loads, so the test is per load.
template <int DT, bool AL>
__device__ __forceinline__ void mask_tail(ItemRaw &r, int lane, int n)
{
    constexpr int E = kE<DT>;
    constexpr uint32_t kNinf = DT == 0 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
__device__ __forceinline__ void lane_vals(const ItemRaw &r, int k, float *x)
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
__device__ __forceinline__ float lane_max(const ItemRaw &r)
{
    constexpr int E = kE<DT>;
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
__device__ __forceinline__ void sample_half(const ItemRaw &r, float c, LaneSum &a, bool first)
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
    float acc[kItemLoads];
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
    for (int w = 1; w < kItemLoads; w <<= 1)
#pragma unroll
        for (int k = 0; k + w < kItemLoads; k += 2 * w) acc[k] += acc[k + w];
    // a lane whose logits are finite but whose sum is not, or a two-part reference: the
    // references move to the lanes' maxima, the earlier sum is rescaled, and the half is
    // summed again (from registers) with the two-part reference when needed
    const bool over = !(acc[0] <= 3.402823466e38f) && fabsf(a.m) <= 3.402823466e38f;
    if (__any(over) || a.huge) {
        const float R = fabsf(a.m) <= 3.402823466e38f ? a.m : 0.0f;
        set_ref(a, R, c);
        a.s = m_prev == -INFINITY ? 0.0f : s_prev * (float)exp2_f64(E_prev - a.E);
        const float Blo = a.huge ? a.Blo : 0.0f;
        float acc2[kItemLoads];
#pragma unroll
        for (int k = 0; k < kItemLoads; ++k) {
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
        for (int w = 1; w < kItemLoads; w <<= 1)
#pragma unroll
            for (int k = 0; k + w < kItemLoads; k += 2 * w) acc2[k] += acc2[k + w];
        acc[0] = acc2[0];
    }
    a.s += acc[0];
    if (a.m == -INFINITY) a.s = 0.0f;
}

// 2^(a/L) in fp64 from a table of the L = 64 values 2^(j/L) in LDS (exp2_tab_read,
// then exp2_tab_finish): a = k + r with
// k = rint(a), so |r| <= 1/2 and 2^(a/L) = 2^floor(k/L) 2^((k mod L)/L) 2^(r/L), with
// 2^(r/L) from its Taylor series in r ln 2 / L to degree 3 (truncation below 4e-11
// relative).  The power 2^floor(k/L) is added to the exponent field of the product,
// which lies in [0.99, 2.02): the caller keeps a >= -1000 L (2^-1000, a term that
// cannot register next to the maximum's 1), so the result stays normal.  Entry j of
// the lane's copy is at col[j << sh] (sh = 6: one column per lane, which no two lanes
// of a wave share, so the reads meet no bank conflicts; sh = 0: a single shared copy).
constexpr int kTabBits = 6;
constexpr int kTabLen = 1 << kTabBits;

struct Exp2Tab {
    const double *col;
    int sh;
};

// (ln 2 / L)^j / j!  (kExp2Coef[13 - j] = (ln 2)^j / j!, scaled by L^-j exactly)
constexpr double kTabC1 = kExp2Coef[12] / kTabLen;
constexpr double kTabC2 = kExp2Coef[11] / kTabLen / kTabLen;
constexpr double kTabC3 = kExp2Coef[10] / kTabLen / kTabLen / kTabLen;

// The two halves of exp2_tab, so that a caller can issue the table reads of several
// terms before it waits for the first: the rounding and the read, then the series.
struct TabTerm {
    double r;   // a - rint(a)
    double T;   // 2^((k mod L)/L)
    int ki;     // rint(a)
};

__device__ __forceinline__ TabTerm exp2_tab_read(double a, const Exp2Tab &t)
{
    const double k = rint(a);
    TabTerm u;
    u.r = a - k;   // exact
    u.ki = (int)k;
    u.T = t.col[(u.ki & (kTabLen - 1)) << t.sh];
    return u;
}

__device__ __forceinline__ double exp2_tab_finish(const TabTerm &u)
{
    const double q = fma(fma(fma(kTabC3, u.r, kTabC2), u.r, kTabC1), u.r, 1.0);
    const double v = u.T * q;
    return __hiloint2double(__double2hiint(v) + (u.ki >> kTabBits) * 1048576, __double2loint(v));
}

// Fill a table of 2^(j/L) for exp2_tab_read: kTabLen entries, each repeated `copies`
// times (64: one column per lane; 1: a single copy).  The caller synchronises after it.
__device__ __forceinline__ void fill_exp2_tab(double *tab, int copies)
{
    for (int i = threadIdx.x; i < kTabLen * copies; i += blockDim.x)
        tab[i] = exp2_f64((double)(i / copies) * (1.0 / kTabLen));
}

// fp32 logits: the sums feed log2(S_t / S_d), which the residual mass of a draft close
// to the target needs to ~1e-9 relative, so every term is an fp64 2^(x c - E): the
// exponent from one fp64 fma (c the full scale), the power from the table.  The half's
// lane maximum comes first and the reference follows the running lane maximum (the
// sum so far rescaled), so every exponent is <= 0 up to rounding.
__device__ __forceinline__ void sample_half_f32(const ItemRaw &r, double c_eff, LaneSum &a, bool first,
                                                const Exp2Tab &tab)
{
    float mh = -INFINITY;
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
    for (int k = 0; k < kItemLoads; ++k) {
        float x[4];
        lane_vals<1, 1>(r, k, x);
        TabTerm u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = exp2_tab_read(fmax(fma((double)x[t], cs, -Es), -1000.0 * kTabLen), tab);
#pragma unroll
        for (int t = 0; t < 4; ++t) s += exp2_tab_finish(u[t]);
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
__device__ __forceinline__ void argmax_half(const ItemRaw &r, int lane, int base, LaneArg &a)
{
    constexpr int E = kE<DT>;
    // per load maximum, then the first load holding the half's lane maximum (strictly
    // greater wins, so the earliest load keeps ties)
    float mh = -INFINITY;
    int kb = 0;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
    for (int k = 1; k < kItemLoads; ++k)
        if (k == kb) w = r.d[k];
    ItemRaw one;
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
__device__ __forceinline__ float half_value(const ItemRaw &r, int lane, int o)
{
    constexpr int E = kE<DT>;
    uint32_t wsel = 0u;
    bool hi = false;
#pragma unroll
    for (int k = 0; k < kItemLoads; ++k) {
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
};

template <int DT, bool AL>
__device__ __forceinline__ void piece_half(const Params &P, const VecCtx &vc, int32_t rm, const TempConst &tc,
                                           int64_t j, int h, int n, ItemRaw &r, PieceAcc<DT> &acc, int lane,
                                           const Exp2Tab &tab)
{
    constexpr int E = kE<DT>;
    if constexpr (!AL) realign(r, lane);
    if (n != (int)P.geo.ie) mask_tail<DT, AL>(r, lane, n);
    if (rm == ROW_SAMPLE) {
        if constexpr (DT == 0) sample_half(r, tc.c_hi, acc.ls, h == 0);
        else sample_half_f32(r, tc.c_eff, acc.ls, h == 0, tab);
        // the logit at the position's draft token, if this half holds it
        if (vc.slot >= 0 && vc.x >= 0 && (int64_t)vc.x < P.V) {
            const int64_t o = (int64_t)vc.x - (2 * j + h) * P.geo.ie;
            if (o >= 0 && o < n) {
                const float z = half_value<DT>(r, lane, (int)o);
                if (lane == (int)((o % (64 * E)) / E)) P.zx[(vc.target ? 0 : P.nD) + vc.slot] = z;
            }
        }
    } else if (rm == ROW_GREEDY && vc.target) {
        if (h == 0) acc.la = LaneArg{-INFINITY, INT32_MAX, false};
        argmax_half<DT>(r, lane, h * (int)P.geo.ie, acc.la);
    }
}

template <int DT>
__device__ __forceinline__ void piece_finish(const Params &P, const VecCtx &vc, int32_t rm, const TempConst &tc,
                                             int64_t v, int64_t j, PieceAcc<DT> &acc)
{
    Partial rec{-INFINITY, INT32_MAX, 0.0};
    if (rm == ROW_SAMPLE) {
        rec = sample_record<DT>(acc.ls, tc.c_hi, tc.c_lo);
    } else if (rm == ROW_GREEDY && vc.target) {
        rec = argmax_record(acc.la);
        if (rec.idx != INT32_MAX) rec.idx += (int32_t)(j * 2 * P.geo.ie);
    }
    if ((threadIdx.x & 63) == 0) P.parts[v * P.geo.ipv + j] = rec;
}

// Workgroup b owns pieces [b N / G, (b + 1) N / G) of the N pieces.  Its waves take
// them in order from a counter in LDS (each wave's first piece is fixed), so a wave
// the CU's arbiter serves less takes fewer pieces and the workgroup's waves finish
// together; with one workgroup per CU the CUs finish together too.
template <int DT, bool AL>
__device__ __forceinline__ void stats_body(const Params &P)
{
    __shared__ uint32_t s_next;
    const int lane = threadIdx.x & 63;
    Exp2Tab tab{nullptr, 6};
    if constexpr (DT == 1) {
        __shared__ double s_tab[kTabLen * 64];
        fill_exp2_tab(s_tab, 64);
        tab.col = s_tab + lane;
    }
    if (threadIdx.x == 0) s_next = 0u;
    __syncthreads();
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const int64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwb = blockDim.x >> 6;
    const int64_t N = P.geo.nitems, G = gridDim.x;
    const int64_t p0 = (int64_t)blockIdx.x * N / G, p1 = ((int64_t)blockIdx.x + 1) * N / G;
    int64_t p = p0 + wave;
    if (p >= p1) return;
    auto grab = [&]() -> int64_t {
        uint32_t t = 0u;
        if (lane == 0) t = atomicAdd(&s_next, 1u);
        return p0 + nwb + (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)t);
    };
    const int64_t ipv = P.geo.ipv;
    int64_t v = qdiv(p, ipv, P.geo.inv_ipv), j = p - v * ipv;
    int64_t pn = grab();   // the piece after this one
    // the two halves of a piece in two register buffers: the next piece's first half
    // is loaded while this piece's second half is reduced, and so on (every load
    // unconditional, no copies between the buffers)
    ItemRaw ra, rb;
    half_begin<DT, AL>(P, v, j, 0, true, ra, lane);
    half_begin<DT, AL>(P, v, j, 1, true, rb, lane);
    VecCtx vc = vec_ctx(P, v);
    float cached_T = __builtin_nanf("");
    TempConst tc{};
    for (;;) {
        const int64_t cv = v, cj = j;
        const bool live = pn < p1;
        int64_t pnn = p1;
        if (live) {
            v = qdiv(pn, ipv, P.geo.inv_ipv);
            j = pn - v * ipv;
            pnn = grab();
        }
        const int32_t rm = row_mode(P.mode, vc.T);
        if (rm == ROW_SAMPLE && vc.T != cached_T) {
            tc = temp_const<DT>(vc.T);
            cached_T = vc.T;
        }
        PieceAcc<DT> acc;
        piece_half<DT, AL>(P, vc, rm, tc, cj, 0, half_len(P, cj, 0), ra, acc, lane, tab);
        half_begin<DT, AL>(P, v, j, 0, live, ra, lane);
        const int n1 = half_len(P, cj, 1);
        if (n1 > 0) piece_half<DT, AL>(P, vc, rm, tc, cj, 1, n1, rb, acc, lane, tab);
        half_begin<DT, AL>(P, v, j, 1, live, rb, lane);
        const VecCtx vn = vec_ctx(P, live ? v : 0);
        piece_finish<DT>(P, vc, rm, tc, cv, cj, acc);
        if (!live) break;
        vc = vn;
        pn = pnn;
    }
}

// One piece of a listed vector per wave: the early-exit steps read only the vectors
// of the rows still undecided at the current position (two list slots per row).
// Workgroup b takes piece b mod ipv of list slot b / ipv; slots past the list's
// length, and holes (-1), do nothing.  Thread 0 of workgroup 0 also clears the other
// list buffer's counts, which the step kernel after this one fills.
template <int DT, bool AL>
__global__ __launch_bounds__(64) void stats_list_kernel(Params P)
{
    const int lane = threadIdx.x;
    const int buf = P.step & 1;
    Exp2Tab tab{nullptr, 0};
    if constexpr (DT == 1) {   // one shared copy: 64 copies would limit the one-wave workgroups per CU
        __shared__ double s_tab[kTabLen];
        fill_exp2_tab(s_tab, 1);
        __syncthreads();
        tab.col = s_tab;
    }
    if (blockIdx.x == 0 && lane == 0) {
        P.ee_count[2 * (buf ^ 1)] = 0;
        P.ee_count[2 * (buf ^ 1) + 1] = 0;
    }
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const int64_t ipv = P.geo.ipv;
    const int64_t slot = (int64_t)blockIdx.x / ipv;
    const int64_t j = (int64_t)blockIdx.x - slot * ipv;
    if (slot >= 2 * (int64_t)P.ee_count[2 * buf]) return;
    const int64_t v = P.ee_vecs[buf][slot];
    if (v < 0) return;
    ItemRaw ra, rb;
    half_begin<DT, AL>(P, v, j, 0, true, ra, lane);
    half_begin<DT, AL>(P, v, j, 1, true, rb, lane);
    const VecCtx vc = vec_ctx(P, v);
    const int32_t rm = row_mode(P.mode, vc.T);
    const TempConst tc = rm == ROW_SAMPLE ? temp_const<DT>(vc.T) : TempConst{};
    PieceAcc<DT> acc;
    piece_half<DT, AL>(P, vc, rm, tc, j, 0, half_len(P, j, 0), ra, acc, lane, tab);
    const int n1 = half_len(P, j, 1);
    if (n1 > 0) piece_half<DT, AL>(P, vc, rm, tc, j, 1, n1, rb, acc, lane, tab);
    piece_finish<DT>(P, vc, rm, tc, v, j, acc);
}

// 16-byte aligned rows (the usual case): one workgroup of 12 waves per CU, 3 per SIMD
template <int DT>
__global__ __launch_bounds__(kStatsBlock) void stats_kernel(Params P)
{
    stats_body<DT, true>(P);
}

// rows that do not start 16-byte aligned: aligned loads, realigned in registers; 8
// waves per CU (the realignment needs registers of its own)
constexpr int kStatsBlockUnaligned = 512;
template <int DT>
__global__ __launch_bounds__(kStatsBlockUnaligned) void stats_kernel_unaligned(Params P)
{
    stats_body<DT, false>(P);
}

// ===========================================================================
// launchers
// ===========================================================================
static hipError_t launch(const void *fn, int64_t blocks, int threads, const Params &P, hipStream_t s)
{
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    void *args[] = {const_cast<Params *>(&P)};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), args, 0, s);
}

static int stats_block(bool aligned) { return aligned ? kStatsBlock : kStatsBlockUnaligned; }

static const void *stats_fn(int dtype, bool aligned)
{
    return dtype == 0 ? (aligned ? (const void *)stats_kernel<0> : (const void *)stats_kernel_unaligned<0>)
                      : (aligned ? (const void *)stats_kernel<1> : (const void *)stats_kernel_unaligned<1>);
}

// Workgroups of the streaming kernel that fit on the current device at once
// (cached per device and kernel variant).
int32_t stats_grid_cap(int dtype, bool aligned)
{
    constexpr int kMaxDev = 64;
    static int32_t cache[kMaxDev][4] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 1024;
    const int var = dtype * 2 + (aligned ? 1 : 0);
    if (dev < kMaxDev && cache[dev][var] > 0) return cache[dev][var];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stats_fn(dtype, aligned), stats_block(aligned), 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 1;
    int64_t cap = (int64_t)cus * per_cu;
    if (cap > kMaxStatsGrid) cap = kMaxStatsGrid;
    if (dev < kMaxDev) cache[dev][var] = (int32_t)cap;
    return (int32_t)cap;
}

hipError_t launch_stats_list(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)stats_list_kernel<0, true> : (const void *)stats_list_kernel<0, false>)
        : (aligned ? (const void *)stats_list_kernel<1, true> : (const void *)stats_list_kernel<1, false>);
    return launch(fn, 2 * (int64_t)P.B * P.geo.ipv, 64, P, s);
}

hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned, hipEvent_t start, hipEvent_t stop)
{
    return launch_timed(stats_fn(dtype, aligned), P.geo.G, stats_block(aligned), P, s, start, stop);
}

}  // namespace sv
