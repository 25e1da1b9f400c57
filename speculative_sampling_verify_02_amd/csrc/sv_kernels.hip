// HIP kernels of the speculative-sampling verification step for gfx950.
//
// stats_kernel streams every logit once.  The vectors it reads (the gamma+1 target
// and gamma draft positions of every row, or only target positions in greedy mode)
// are laid end to end and cut into equal contiguous pieces, one per workgroup, so
// every workgroup does the same work and the grid ends together.  For each
// (workgroup, vector) overlap it writes the maximum and the sum of exp((z - m)/T)
// (sampling rows) or the first argmax (greedy rows).  The temperature softmax these
// summarize is the softened output of brunomaga.github.io "inference-distillation-
// speculative-decoding", section "Knowledge distillation", with one T for both
// models (rayaq.ca "Speculative decoding", section "Why the output is exactly the
// target's").
//
// verify_kernel gives each row one wave for the accept scan: it merges the pieces,
// computes p(x_j) and q(x_j), and keeps x_j while u_j < min(1, p_j(x_j)/q_j(x_j))
// (rayaq.ca "Speculative decoding", section "One round", step 3), or while x_j
// equals the argmax in greedy mode (section "The greedy case").  The workgroups of a
// sampling row then re-read only position K and sum the draw weights per 512-logit
// tile: the residual max(0, p - q) after a rejection (step 4) or p for the bonus
// token (step 5).  draw_final_kernel walks one row's tile sums and one tile to the
// inverse-CDF token.
//
// bf16 logits are processed in fp32 (exp2 on the hardware unit, fp64 accumulation
// of 8-logit partial sums); fp32 logits are processed in fp64 throughout.
#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

constexpr double kQNaN = __builtin_nan("");

// ===========================================================================
// prepare: packed offsets of a ragged batch
// ===========================================================================
__global__ __launch_bounds__(1024) void prepare_kernel(Params P)
{
    __shared__ int64_t sh_t[16], sh_d[16];
    __shared__ int64_t carry_t, carry_d;
    __shared__ int bad;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry_t = carry_d = 0;
        bad = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < P.B; base += 1024) {
        const int64_t i = base + tid;
        const bool in = i < P.B;
        int32_t g = in ? P.gamma[i] : 0;
        if (in && g < 0) bad = 1;
        if (g < 0) g = 0;
        const int64_t vt = in ? (int64_t)g + 1 : 0, vd = in ? (int64_t)g : 0;
        int64_t it = vt, id = vd;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t a = __shfl_up(it, o), b = __shfl_up(id, o);
            if (lane >= o) { it += a; id += b; }
        }
        if (lane == 63) { sh_t[wave] = it; sh_d[wave] = id; }
        __syncthreads();
        int64_t pt = carry_t, pd = carry_d;
        for (int w = 0; w < wave; ++w) { pt += sh_t[w]; pd += sh_d[w]; }
        const int64_t t_off = pt + it - vt, d_off = pd + id - vd;
        if (in) {
            P.rows[i] = RowInfo{(int32_t)t_off, (int32_t)d_off, g, 0};
            // streamed slots of row i (bounds-checked: totals are validated below)
            const int64_t s0 = P.mode == 1 ? t_off : t_off + d_off;
            const int64_t n = P.mode == 1 ? (int64_t)g + 1 : 2 * (int64_t)g + 1;
            if (s0 < P.geo.nvec) {
                const int64_t e = s0 + n < P.geo.nvec ? s0 + n : P.geo.nvec;
                for (int64_t k = s0; k < e; ++k) P.vec_row[k] = (int32_t)i;
            }
        }
        __syncthreads();
        if (tid == 1023) { carry_t = pt + it; carry_d = pd + id; }
        __syncthreads();
    }
    if (tid == 0) P.hdr->status = (bad || carry_t != P.nT) ? ST_BAD_GAMMA : 0;
}

// ===========================================================================
// streaming pass
// ===========================================================================

// Sampling accumulator of one thread, fp32 arithmetic (bf16 logits).  s holds
// sum 2^(z c - R) against an integer reference R, or, on the slow route (scaled
// logits at or beyond 2^20 in magnitude), sum 2^((z - mref) c).  R moves to the
// smallest integer at or above a group's scaled maximum when that maximum passes
// it, an exact power-of-two rescale of s, so the largest terms have arguments in
// (-1, 0].  Before any finite logit R = 0 and has_ref is false: -inf logits add 0
// and a NaN logit makes s NaN.  Rare paths sit behind wave-uniform branches.
struct Acc32 {
    float m;        // running maximum
    float R;        // integer reference (fast route)
    float mref;     // reference logit (slow route)
    bool has_ref;
    bool slow;
    double s;
};

template <int N>
__device__ __forceinline__ void acc32_group(Acc32 &a, const float *x, const TempConst &tc)
{
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) cm = __builtin_elementwise_maximum(cm, x[i]);
    a.m = __builtin_elementwise_maximum(a.m, cm);
    const bool up = a.slow ? cm > a.mref : (cm * tc.c_hi > a.R || (!a.has_ref && cm > -INFINITY));
    if (__any(up)) {
        if (up) {
            const float Rn = ceilf(cm * tc.c_hi);
            const bool slow = !(fabsf(Rn) < kFastRef);
            if (a.has_ref) {
                if (!a.slow && !slow) {
                    a.s = ldexp(a.s, (int)(a.R - Rn));
                } else {
                    const double Rold = a.slow ? (double)a.mref * tc.c_eff : (double)a.R;
                    const double Rnew = slow ? (double)cm * tc.c_eff : (double)Rn;
                    a.s *= exp2_f64(Rold - Rnew);
                }
            }
            a.R = slow ? 0.0f : Rn;
            a.mref = cm;
            a.slow = slow;
            a.has_ref = true;
        }
    }
    float e[N];
    if (__any(a.slow)) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float d = x[i] - a.mref;
            const float es = hw_exp2(fmaf(d, tc.c_hi, d * tc.c_lo));
            const float ef = hw_exp2(fmaf(x[i], tc.c_lo, fmaf(x[i], tc.c_hi, -a.R)));
            e[i] = a.slow ? es : ef;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) e[i] = hw_exp2(fmaf(x[i], tc.c_lo, fmaf(x[i], tc.c_hi, -a.R)));
    }
#pragma unroll
    for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
    a.s += (double)e[0];
}

// this thread's sum relative to its own maximum m: sum 2^((z - m) c)
__device__ __forceinline__ double acc32_final(const Acc32 &a, const TempConst &tc)
{
    if (!a.has_ref) return a.s;   // 0, or NaN
    const double Rd = a.slow ? (double)a.mref * tc.c_eff : (double)a.R;
    return a.s * exp2_f64(Rd - (double)a.m * tc.c_eff);
}

// Sampling accumulator in fp64 (fp32 logits), same scheme with an fp64 reference.
struct Acc64 {
    float m;
    bool has_ref;
    double R;
    double s;
};

template <int N>
__device__ __forceinline__ void acc64_group(Acc64 &a, const float *x, const TempConst &tc)
{
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) cm = __builtin_elementwise_maximum(cm, x[i]);
    a.m = __builtin_elementwise_maximum(a.m, cm);
    const double sc = (double)cm * tc.c_eff;
    const bool up = sc > a.R || (!a.has_ref && cm > -INFINITY);
    if (__any(up)) {
        if (up) {
            const double Rn = ceil(sc);
            if (a.has_ref) {
                const double sh = a.R - Rn;
                a.s = sh < -2000.0 ? a.s * 0.0 : ldexp(a.s, (int)sh);
            }
            a.R = Rn;
            a.has_ref = true;
        }
    }
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < N; ++i) t += exp2_f64(fma((double)x[i], tc.c_eff, -a.R));
    a.s += t;
}

__device__ __forceinline__ double acc64_final(const Acc64 &a, const TempConst &tc)
{
    if (!a.has_ref) return a.s;
    return a.s * exp2_f64(a.R - (double)a.m * tc.c_eff);
}

struct AccArg {
    float best;
    int32_t idx;
    bool nan_seen;
};

// x holds kUnroll units, unit k at index u + k * kBlock
template <int N>
__device__ __forceinline__ void accarg_group(AccArg &a, const float *x, int64_t u)
{
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) cm = __builtin_elementwise_maximum(cm, x[i]);
    bool nan = false;
#pragma unroll
    for (int i = 0; i < N; ++i) nan |= (x[i] != x[i]);
    a.nan_seen |= nan;
    const bool up = cm > a.best;
    if (__any(up)) {
        if (up) {
            a.best = cm;
            int first = N - 1;
#pragma unroll
            for (int i = N - 1; i >= 0; --i)
                if (x[i] == cm) first = i;
            a.idx = (int32_t)((u + (int64_t)(first / kUnitElems) * kBlock) * kUnitElems + first % kUnitElems);
        }
    }
}

// A unit past the end of the piece, read as -inf logits.
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

// One vector piece [a, b) (units) by the whole workgroup.
template <int DT, bool AL>
__device__ Partial reduce_piece(const void *base, int64_t a, int64_t b, int64_t V, int rmode,
                                const TempConst &tc)
{
    constexpr int kHalf = kUnroll / 2 * kUnitElems;
    __shared__ float sh_f[kWaves];
    __shared__ double sh_d[kWaves];
    __shared__ int sh_i[kWaves], sh_n[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __syncthreads();   // the shared slots may still be read by a previous piece

    Acc32 a32{-INFINITY, 0.0f, 0.0f, false, false, 0.0};
    Acc64 a64{-INFINITY, false, 0.0, 0.0};
    AccArg ag{-INFINITY, INT32_MAX, false};

    // one group = kUnroll units per thread, unit k of thread t at u + t + k * kBlock
    auto group = [&](const RawUnit<DT> *r, int64_t u) {
        // two halves of kHalf logits each keep fewer values live at once
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float x[kHalf];
#pragma unroll
            for (int k = 0; k < kUnroll / 2; ++k) unpack<DT>(r[h * (kUnroll / 2) + k], x + k * kUnitElems);
            if (rmode == ROW_GREEDY) accarg_group<kHalf>(ag, x, u + (int64_t)h * (kUnroll / 2) * kBlock);
            else if (DT == 0) acc32_group<kHalf>(a32, x, tc);
            else acc64_group<kHalf>(a64, x, tc);
        }
    };

    constexpr int64_t kStride = (int64_t)kBlock * kUnroll;
    constexpr uint32_t kUnitBytes = DT == 0 ? 16u : 32u;
    int64_t u_tail = a;   // first group start not covered by the unpredicated loop
    if constexpr (AL) {
        // full groups: unpredicated buffer loads at 32-bit offsets from the piece
        // start, the next group's loads in flight while this one is reduced
        // (an fp32 vector whose length is not a multiple of 8 ends in a partial unit;
        // that unit is left to the predicated loop)
        const int64_t n = b - a - ((DT == 1 && b * kUnitElems > V) ? 1 : 0);
        const int64_t nfull = n / kStride;
        if (nfull > 0 && n * kUnitBytes < ((int64_t)1 << 31)) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(static_cast<const char *>(base) + a * kUnitBytes), 0,
                (int)(n * kUnitBytes), kBufferWord3);
            auto load_group = [&](RawUnit<DT> *r, uint32_t off) {
#pragma unroll
                for (int k = 0; k < kUnroll; ++k) r[k] = buffer_unit<DT>(rs, off + (uint32_t)k * kBlock * kUnitBytes);
            };
            // two alternating register buffers (no copies between them, so waiting for
            // one group's loads leaves the next group's loads in flight)
            const uint32_t off0 = (uint32_t)tid * kUnitBytes;
            const uint32_t step = (uint32_t)kStride * kUnitBytes;
            RawUnit<DT> ra[kUnroll], rb[kUnroll];
            load_group(ra, off0);
            int64_t it = 0;
            for (; it + 2 < nfull; it += 2) {   // prefetches always in range here
                load_group(rb, off0 + (uint32_t)(it + 1) * step);
                group(ra, a + it * kStride + tid);
                load_group(ra, off0 + (uint32_t)(it + 2) * step);
                group(rb, a + (it + 1) * kStride + tid);
            }
            if (it + 1 < nfull) {
                load_group(rb, off0 + (uint32_t)(it + 1) * step);
                group(ra, a + it * kStride + tid);
                group(rb, a + (it + 1) * kStride + tid);
            } else {
                group(ra, a + it * kStride + tid);
            }
            u_tail = a + nfull * kStride;
        }
    }
    // remaining units, predicated (logits past b read as -inf)
    for (int64_t u = u_tail + tid; u - tid < b; u += kStride) {
        RawUnit<DT> r[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t uk = u + (int64_t)k * kBlock;
            r[k] = uk < b ? load_raw<DT, AL>(base, uk, V) : neg_inf_unit<DT>();
        }
        group(r, u);
    }

    Partial out;
    if (rmode == ROW_GREEDY) {
        float bst = wave_max(ag.best);
        if (lane == 0) sh_f[wave] = bst;
        __syncthreads();
        bst = fmaxf(fmaxf(sh_f[0], sh_f[1]), fmaxf(sh_f[2], sh_f[3]));
        int cand = wave_min_int(ag.best == bst ? ag.idx : INT32_MAX);
        const int nan = wave_or_int(ag.nan_seen ? 1 : 0);
        if (lane == 0) { sh_i[wave] = cand; sh_n[wave] = nan; }
        __syncthreads();
        out.m = bst;
        out.idx = min(min(sh_i[0], sh_i[1]), min(sh_i[2], sh_i[3]));
        out.s = (sh_n[0] | sh_n[1] | sh_n[2] | sh_n[3]) ? kQNaN : 0.0;
        return out;
    }
    // this thread's sum relative to its own maximum, then the workgroup's
    const float m = DT == 0 ? a32.m : a64.m;
    const double s_m = DT == 0 ? acc32_final(a32, tc) : acc64_final(a64, tc);
    float mw = wave_max(m);
    if (lane == 0) sh_f[wave] = mw;
    __syncthreads();
    mw = fmaxf(fmaxf(sh_f[0], sh_f[1]), fmaxf(sh_f[2], sh_f[3]));
    double c = (m == -INFINITY) ? s_m : s_m * exp2_f64(((double)m - (double)mw) * tc.c_eff);
    c = wave_sum(c);
    if (lane == 0) sh_d[wave] = c;
    __syncthreads();
    out.m = mw;
    out.idx = 0;
    out.s = (sh_d[0] + sh_d[1]) + (sh_d[2] + sh_d[3]);
    return out;
}

__device__ __forceinline__ int32_t slot_row(const Params &P, int64_t v)
{
    if (P.gamma != nullptr) return P.vec_row[v];
    const int64_t per = P.mode == 1 ? (int64_t)P.gamma_uniform + 1 : 2 * (int64_t)P.gamma_uniform + 1;
    return (int32_t)(v / per);
}

template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void stats_kernel(Params P)
{
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const int64_t wg = blockIdx.x;
    const int64_t nunits = P.geo.nunits;
    const int64_t u0 = wg * P.geo.R;
    int64_t u1 = u0 + P.geo.R;
    if (u1 > P.geo.total_units) u1 = P.geo.total_units;
    if (u0 >= u1) return;
    const int64_t v0 = u0 / nunits, v1 = (u1 - 1) / nunits;
    for (int64_t v = v0; v <= v1; ++v) {
        const int64_t vb = v * nunits;
        const int64_t a = (u0 > vb ? u0 : vb) - vb;
        const int64_t b = (u1 < vb + nunits ? u1 : vb + nunits) - vb;
        const int32_t row = slot_row(P, v);
        const RowGeom G = row_geom(P, row);
        const int64_t k = v - row_slot0(P, G);
        const bool is_target = P.mode == 1 || k <= G.gamma;
        const int64_t vrow = is_target ? G.t_off + k : G.d_off + (k - G.gamma - 1);
        const float T = P.temperature[row];
        const int32_t rm = row_mode(P.mode, T);
        Partial rec{-INFINITY, INT32_MAX, 0.0};
        if (rm != ROW_BAD_TEMP && (rm == ROW_SAMPLE || is_target)) {
            const TempConst tc = temp_const(rm == ROW_SAMPLE ? T : 1.0f);
            const void *base = vec_ptr(is_target ? P.target : P.draft, DT, vrow, P.V);
            // the logit at this position's draft token, if it lies in this piece
            // (sampling rows), saved for the accept test
            const int64_t j = is_target ? k : k - G.gamma - 1;
            float zx = 0.0f;
            bool have_zx = false;
            if (rm == ROW_SAMPLE && j < G.gamma) {
                const int32_t x = P.tokens[G.d_off + j];
                if (x >= 0 && (int64_t)x < P.V && x / kUnitElems >= a && x / kUnitElems < b) {
                    zx = load_logit<DT>(base, x);
                    have_zx = true;
                }
            }
            rec = reduce_piece<DT, AL>(base, a, b, P.V, rm, tc);
            if (have_zx && threadIdx.x == 0) P.zx[(is_target ? 0 : P.nD) + G.d_off + j] = zx;
        }
        if (threadIdx.x == 0) P.parts[wg + v] = rec;
    }
}

// ===========================================================================
// accept scan: one wave per row
// ===========================================================================
constexpr int kPre = 4;   // pieces of a vector fetched up front (more are fetched later)

struct VecRecs {
    Partial r[kPre];
    int64_t v, w0, w1;    // streamed vector, first and last workgroup whose piece covers it
};

__device__ __forceinline__ void fetch_recs(const Params &P, int64_t v, VecRecs &R)
{
    R.v = v;
    R.w0 = (v * P.geo.nunits) / P.geo.R;
    R.w1 = ((v + 1) * P.geo.nunits - 1) / P.geo.R;
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        R.r[i] = (R.w0 + i <= R.w1) ? P.parts[R.w0 + i + v] : Partial{-INFINITY, INT32_MAX, 0.0};
}

__device__ __forceinline__ void merge_one(const Partial &q, bool greedy, const TempConst &tc, float &m,
                                          double &S, int32_t &idx, bool &nan)
{
    if (greedy) {
        if (q.m > m) {
            m = q.m;
            idx = q.idx;
        } else if (q.m == m && q.idx < idx) {
            idx = q.idx;
        }
        nan |= (q.s != q.s);
        return;
    }
    if (q.m > m) {
        if (m != -INFINITY) S *= exp2_f64(((double)m - (double)q.m) * tc.c_eff);
        m = q.m;
    }
    S += q.m == -INFINITY ? q.s : q.s * exp2_f64(((double)q.m - (double)m) * tc.c_eff);
}

// merge the pieces of a vector: max and sum 2^((z - m) c), or first argmax
__device__ __forceinline__ void merge_recs(const Params &P, const VecRecs &R, const TempConst &tc, bool greedy,
                                           float &m, double &S, int32_t &idx, bool &nan)
{
    m = -INFINITY;
    S = 0.0;
    idx = INT32_MAX;
    nan = false;
#pragma unroll
    for (int i = 0; i < kPre; ++i) merge_one(R.r[i], greedy, tc, m, S, idx, nan);
    for (int64_t w = R.w0 + kPre; w <= R.w1; ++w) merge_one(P.parts[w + R.v], greedy, tc, m, S, idx, nan);
}

// The accept scan of one row by one wave (positions across lanes).  Returns what
// the draw needs (identical on every lane); with `write`, also stores the row's
// outputs.
template <int DT>
__device__ RowDraw scan_row(const Params &P, int32_t row, bool write)
{
    const int lane = threadIdx.x & 63;
    const RowGeom G = row_geom(P, row);
    const int32_t g = G.gamma;
    const int64_t slot0 = row_slot0(P, G);
    const float T = P.temperature[row];
    const int32_t rm = row_mode(P.mode, T);
    const bool greedy = rm == ROW_GREEDY;
    int status = (rm == ROW_BAD_TEMP) ? ST_BAD_TEMP : 0;
    int32_t K = g;
    bool found = false;
    float kmt = -INFINITY, kmd = -INFINITY;   // statistics at K (on every lane once known)
    double kSt = 0.0, kSd = 0.0;
    int32_t kidx = -1;
    int32_t x_keep = 0;                       // this lane's draft token (rows with gamma < 64)

    if (rm != ROW_BAD_TEMP) {
        for (int base = 0; base <= g; base += 64) {
            const int j = base + lane;
            const bool has_t = j <= g, has_d = j < g;
            // every load of this chunk first
            int32_t x = 0;
            float u = 0.0f, zt = 0.0f, zd = 0.0f;
            VecRecs rt, rd;
            if (has_t) fetch_recs(P, slot0 + j, rt);
            if (has_d) {
                x = P.tokens[G.d_off + j];
                u = P.uniforms[G.t_off + j];
                if (!greedy) {   // saved by the streaming pass
                    zt = P.zx[G.d_off + j];
                    zd = P.zx[P.nD + G.d_off + j];
                    fetch_recs(P, slot0 + g + 1 + j, rd);
                }
            }
            x_keep = x;
            const TempConst tc = temp_const(rm == ROW_SAMPLE ? T : 1.0f);
            const bool x_ok = x >= 0 && (int64_t)x < P.V;
            if (has_d && !x_ok) status |= ST_BAD_TOKEN;
            float mt = -INFINITY, md = -INFINITY;
            double St = 0.0, Sd = 0.0;
            int32_t it = INT32_MAX, idd;
            bool nt = false, nd = false;
            bool reject = false;
            if (has_t) merge_recs(P, rt, tc, greedy, mt, St, it, nt);
            if (greedy) {
                if (has_t && (nt || !(mt > -INFINITY && mt < INFINITY))) status |= ST_NONFINITE;
                if (has_d) reject = x != it;
            } else {
                if (has_t && !(St > 0.0 && St < INFINITY)) status |= ST_NONFINITE;
                if (has_d) {
                    merge_recs(P, rd, tc, false, md, Sd, idd, nd);
                    if (!(Sd > 0.0 && Sd < INFINITY)) status |= ST_NONFINITE;
                    double px = kQNaN, qx = kQNaN;
                    if (x_ok && St > 0.0 && St < INFINITY && Sd > 0.0 && Sd < INFINITY) {
                        const double Td = (double)T;
                        px = exp(((double)zt - (double)mt) / Td) / St;
                        qx = exp(((double)zd - (double)md) / Td) / Sd;
                        double ratio;
                        if (qx > 0.0) {
                            ratio = px / qx;
                            if (ratio > 1.0) ratio = 1.0;
                        } else {
                            ratio = px > 0.0 ? 1.0 : 0.0;
                            status |= ST_Q_ZERO;
                        }
                        reject = !((double)u < ratio);
                    }
                    if (write) {
                        if (P.p_x) P.p_x[G.d_off + j] = px;
                        if (P.q_x) P.q_x[G.d_off + j] = qx;
                    }
                }
            }
            const unsigned long long rb = __ballot(reject);
            int src = -1;
            if (!found && rb != 0ull) {
                src = __ffsll((long long)rb) - 1;
                K = base + src;
                found = true;
            } else if (!found && g - base < 64) {
                src = g - base;   // no rejection: the bonus position is in this chunk
            }
            if (src >= 0) {
                kmt = __shfl(mt, src);
                kSt = __shfl(St, src);
                kmd = __shfl(md, src);
                kSd = __shfl(Sd, src);
                kidx = __shfl(it, src);
            }
        }
    }
    status = wave_or_int(status);
    const bool invalid = (status & ST_INVALID) != 0;

    RowDraw D{};
    D.kind = DRAW_NONE;
    if (!invalid && !greedy) {
        D.kind = K < g ? DRAW_RESIDUAL : DRAW_BONUS;
        D.K = K;
        D.t_row = (int32_t)(G.t_off + K);
        D.d_row = (int32_t)(G.d_off + K);
        D.u = P.uniforms[G.t_off + g];
        D.t_slot = (int32_t)(G.t_off + K);
        D.m_t = kmt;
        D.S_t = kSt;
        D.m_d = kmd;
        D.S_d = kSd;
        D.T = T;
    }
    if (write) {
        for (int j = lane; j <= g; j += 64) {
            int32_t e = -1;
            if (!invalid) {
                if (j < K) e = g < 64 ? x_keep : P.tokens[G.d_off + j];
                else if (j == K && greedy) e = kidx;
            }
            P.emitted[G.t_off + j] = e;
            if (j < g && (invalid || greedy)) {
                if (P.p_x) P.p_x[G.d_off + j] = kQNaN;
                if (P.q_x) P.q_x[G.d_off + j] = kQNaN;
            }
        }
        if (lane == 0) {
            P.n_accepted[row] = invalid ? -1 : K;
            if (P.row_status) P.row_status[row] = status;
            if (D.kind == DRAW_NONE && P.resid) P.resid[row] = kQNaN;
            P.draws[row] = D;
        }
    }
    return D;
}

// Ragged batch whose gamma array is inconsistent: every row and slot is invalid.
__device__ void invalidate_call(const Params &P, int32_t row, bool row_writer)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t s = gid; s < P.nT; s += nthreads) P.emitted[s] = -1;
    for (int64_t s = gid; s < P.nD; s += nthreads) {
        if (P.p_x) P.p_x[s] = kQNaN;
        if (P.q_x) P.q_x[s] = kQNaN;
    }
    if (row_writer && row < P.B) {
        P.n_accepted[row] = -1;
        if (P.row_status) P.row_status[row] = ST_BAD_GAMMA;
        if (P.resid) P.resid[row] = kQNaN;
        P.draws[row].kind = DRAW_NONE;
    }
}

// ===========================================================================
// draw: per-tile weight sums, then the inverse CDF
// ===========================================================================
template <int DT>
struct DrawConst;

// bf16 logits: fp32 weights against an integer reference (as in the streaming pass)
template <>
struct DrawConst<0> {
    TempConst tc;
    float Rt, Rd, mt, md, Ft, Fd;
    bool slow_t, slow_d, residual;

    __device__ __forceinline__ void init(const RowDraw &D)
    {
        tc = temp_const(D.T);
        residual = D.kind == DRAW_RESIDUAL;
        mt = D.m_t;
        Rt = ceilf(mt * tc.c_hi);
        slow_t = !(fabsf(Rt) < kFastRef);
        Ft = (float)((slow_t ? 1.0 : exp2_f64((double)Rt - (double)mt * tc.c_eff)) / D.S_t);
        md = D.m_d;
        Rd = ceilf(md * tc.c_hi);
        slow_d = !(fabsf(Rd) < kFastRef);
        Fd = residual ? (float)((slow_d ? 1.0 : exp2_f64((double)Rd - (double)md * tc.c_eff)) / D.S_d) : 0.0f;
    }
    __device__ __forceinline__ float unnorm(float z, float R, float m, bool slow) const
    {
        if (!slow) return hw_exp2(fmaf(z, tc.c_lo, fmaf(z, tc.c_hi, -R)));
        const float d = z - m;
        return hw_exp2(fmaf(d, tc.c_hi, d * tc.c_lo));
    }
    // weights of one unit: w (residual or p) and p, as doubles
    __device__ __forceinline__ void weights(const float *zt, const float *zd, double *w, double *p) const
    {
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const float pe = unnorm(zt[e], Rt, mt, slow_t) * Ft;
            float we = pe;
            if (residual) we = fmaxf(0.0f, pe - unnorm(zd[e], Rd, md, slow_d) * Fd);
            w[e] = we;
            p[e] = pe;
        }
    }
};

// fp32 logits: fp64 weights
template <>
struct DrawConst<1> {
    TempConst tc;
    double Rt, Rd, Ft, Fd;
    bool residual;

    __device__ __forceinline__ void init(const RowDraw &D)
    {
        tc = temp_const(D.T);
        residual = D.kind == DRAW_RESIDUAL;
        Rt = ceil((double)D.m_t * tc.c_eff);
        Ft = exp2_f64(Rt - (double)D.m_t * tc.c_eff) / D.S_t;
        Rd = residual ? ceil((double)D.m_d * tc.c_eff) : 0.0;
        Fd = residual ? exp2_f64(Rd - (double)D.m_d * tc.c_eff) / D.S_d : 0.0;
    }
    __device__ __forceinline__ void weights(const float *zt, const float *zd, double *w, double *p) const
    {
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const double pe = exp2_f64(fma((double)zt[e], tc.c_eff, -Rt)) * Ft;
            double we = pe;
            if (residual) we = fmax(0.0, pe - exp2_f64(fma((double)zd[e], tc.c_eff, -Rd)) * Fd);
            w[e] = we;
            p[e] = pe;
        }
    }
};

template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void verify_kernel(Params P)
{
    __shared__ RowDraw sD;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per_row = P.mode == 1 ? 1 : P.geo.ndraw;
    const int32_t row = (int32_t)(blockIdx.x / per_row);
    const int32_t piece = (int32_t)(blockIdx.x - (int64_t)row * per_row);
    if (P.gamma != nullptr && P.hdr->status != 0) {
        invalidate_call(P, row, piece == 0 && tid == 0);
        return;
    }
    // every workgroup of the row runs the scan (a few hundred bytes from L2); the
    // first one stores the row's outputs
    if (wave == 0) {
        const RowDraw d = scan_row<DT>(P, row, piece == 0);
        if (lane == 0) sD = d;
    }
    __syncthreads();
    const RowDraw D = sD;
    if (D.kind == DRAW_NONE) return;
    DrawConst<DT> c;
    c.init(D);
    const void *tb = vec_ptr(P.target, DT, D.t_row, P.V);
    const void *db = c.residual ? vec_ptr(P.draft, DT, D.d_row, P.V) : nullptr;
    const int64_t t0 = (int64_t)piece * kTilesPerDrawWg + (int64_t)wave * kTilesPerWave;

    RawUnit<DT> rt[kTilesPerWave], rd[kTilesPerWave];
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        const int64_t unit = (t0 + i) * kTileUnits + lane;
        const bool in = t0 + i < P.geo.ntiles && unit < P.geo.nunits;
        rt[i] = in ? load_raw<DT, AL>(tb, unit, P.V) : neg_inf_unit<DT>();
        rd[i] = (in && c.residual) ? load_raw<DT, AL>(db, unit, P.V) : neg_inf_unit<DT>();
    }
    // per-lane sums of every tile first, then one interleaved cross-lane reduction
    // (tiles past the end read -inf logits and sum to 0)
    double lw[kTilesPerWave], lp[kTilesPerWave];
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        float zt[kUnitElems], zd[kUnitElems];
        unpack<DT>(rt[i], zt);
        unpack<DT>(rd[i], zd);
        double w[kUnitElems], p[kUnitElems];
        c.weights(zt, zd, w, p);
        lw[i] = 0.0;
        lp[i] = 0.0;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) { lw[i] += w[e]; lp[i] += p[e]; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            lw[i] += __shfl_xor(lw[i], o);
            lp[i] += __shfl_xor(lp[i], o);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i)
            if (t0 + i < P.geo.ntiles) P.tiles[row * P.geo.ntiles + t0 + i] = Sum2{lw[i], lp[i]};
    }
}

// one wave per row
template <int DT, bool AL>
__global__ __launch_bounds__(64) void draw_final_kernel(Params P)
{
    const int lane = threadIdx.x;
    const int32_t row = blockIdx.x;
    const RowDraw D = P.draws[row];
    if (D.kind == DRAW_NONE) return;
    const int32_t nt = P.geo.ntiles;
    const Sum2 *tiles = P.tiles + (int64_t)row * nt;
    const int per = (nt + 63) / 64;        // tiles per lane, contiguous
    const int l0 = lane * per;
    const int l1 = min(l0 + per, nt);

    // total weight (residual, or p when the residual is empty)
    double lw = 0.0, lp = 0.0;
    for (int t = l0; t < l1; ++t) { lw += tiles[t].w; lp += tiles[t].p; }
    const double iw = wave_inclusive_sum(lw, lane), ip = wave_inclusive_sum(lp, lane);
    double W = __shfl(iw, 63);
    bool use_p = false;
    if (D.kind == DRAW_RESIDUAL && !(W > 0.0)) use_p = true;
    if (D.kind == DRAW_BONUS) use_p = false;
    if (use_p) W = __shfl(ip, 63);
    const double t = (double)D.u * W;

    // the tile where the running sum first exceeds t
    double cum = use_p ? ip - lp : iw - lw;
    int cand = -1, lastpos = -1;
    double cand_before = 0.0, last_before = 0.0;
    for (int k = l0; k < l1; ++k) {
        const double v = use_p ? tiles[k].p : tiles[k].w;
        if (cand < 0 && cum + v > t) { cand = k; cand_before = cum; }
        if (v > 0.0) { lastpos = k; last_before = cum; }
        cum += v;
    }
    int tile = -1;
    double before = 0.0;
    const unsigned long long hit = __ballot(cand >= 0);
    if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        tile = __shfl(cand, l);
        before = __shfl(cand_before, l);
    } else {
        const unsigned long long pos = __ballot(lastpos >= 0);
        if (pos) {
            const int l = 63 - __clzll((long long)pos);
            tile = __shfl(lastpos, l);
            before = __shfl(last_before, l);
        }
    }

    int32_t token = -1;
    if (tile >= 0) {
        DrawConst<DT> c;
        c.init(D);
        const void *tb = vec_ptr(P.target, DT, D.t_row, P.V);
        const void *db = c.residual ? vec_ptr(P.draft, DT, D.d_row, P.V) : nullptr;
        const int64_t unit = (int64_t)tile * kTileUnits + lane;
        const bool in = unit < P.geo.nunits;
        const RawUnit<DT> rt = in ? load_raw<DT, AL>(tb, unit, P.V) : neg_inf_unit<DT>();
        const RawUnit<DT> rd = (in && c.residual) ? load_raw<DT, AL>(db, unit, P.V) : neg_inf_unit<DT>();
        float zt[kUnitElems], zd[kUnitElems];
        unpack<DT>(rt, zt);
        unpack<DT>(rd, zd);
        double w[kUnitElems], p[kUnitElems];
        c.weights(zt, zd, w, p);
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) ls += use_p ? p[e] : w[e];
        const double incl = wave_inclusive_sum(ls, lane);
        double run = before + incl - ls;
        int ce = -1, lpos = -1;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const double we = use_p ? p[e] : w[e];
            run += we;
            if (ce < 0 && run > t) ce = e;
            if (we > 0.0) lpos = e;
        }
        const unsigned long long h2 = __ballot(ce >= 0);
        if (h2) {
            const int l = __ffsll((long long)h2) - 1;
            token = __shfl((int)(unit * kUnitElems) + ce, l);
        } else {
            const unsigned long long p2 = __ballot(lpos >= 0);
            if (p2) {
                const int l = 63 - __clzll((long long)p2);
                token = __shfl((int)(unit * kUnitElems) + lpos, l);
            }
        }
    }
    if (lane == 0) {
        P.emitted[D.t_slot] = token;
        if (P.resid) P.resid[row] = W;
        if (use_p && P.row_status) P.row_status[row] |= ST_ZERO_RESID;
    }
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

static const void *stats_fn(int dtype, bool aligned)
{
    return dtype == 0 ? (aligned ? (const void *)stats_kernel<0, true> : (const void *)stats_kernel<0, false>)
                      : (aligned ? (const void *)stats_kernel<1, true> : (const void *)stats_kernel<1, false>);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stats_fn(dtype, aligned), kBlock, 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 4;
    int64_t cap = (int64_t)cus * per_cu;
    if (cap > kMaxStatsGrid) cap = kMaxStatsGrid;
    if (dev < kMaxDev) cache[dev][var] = (int32_t)cap;
    return (int32_t)cap;
}

hipError_t launch_prepare(const Params &P, hipStream_t s)
{
    return launch((const void *)prepare_kernel, 1, 1024, P, s);
}

hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    return launch(stats_fn(dtype, aligned), P.geo.G, kBlock, P, s);
}

hipError_t launch_verify(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)verify_kernel<0, true> : (const void *)verify_kernel<0, false>)
        : (aligned ? (const void *)verify_kernel<1, true> : (const void *)verify_kernel<1, false>);
    const int64_t per_row = P.mode == 1 ? 1 : P.geo.ndraw;
    return launch(fn, (int64_t)P.B * per_row, kBlock, P, s);
}

hipError_t launch_draw_final(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)draw_final_kernel<0, true> : (const void *)draw_final_kernel<0, false>)
        : (aligned ? (const void *)draw_final_kernel<1, true> : (const void *)draw_final_kernel<1, false>);
    return launch(fn, P.B, 64, P, s);
}

}  // namespace sv
