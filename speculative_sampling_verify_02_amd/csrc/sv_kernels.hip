// HIP kernels of the speculative-sampling verification step for gfx950.
//
// Pass 1 (stats_kernel) streams every logit once: for every (row, position) vector
// it produces the maximum and the sum of exp((z - m)/T) (sampling rows) or the first
// argmax (greedy rows), split over a few segments per vector so the grid has
// thousands of workgroups.  The temperature softmax it summarizes is the softened
// output of brunomaga.github.io "inference-distillation-speculative-decoding",
// section "Knowledge distillation", applied with one T to both models (rayaq.ca
// "Speculative decoding", section "Why the output is exactly the target's").
//
// The accept scan (scan_kernel) walks each row left to right, keeping x_j while
// u_j < min(1, p_j(x_j)/q_j(x_j)) (rayaq.ca "Speculative decoding", section "One
// round", step 3), or while x_j equals the argmax in greedy mode (section "The
// greedy case").
//
// Pass 2 (draw_kernel) re-reads only the position K of each sampling row: the
// residual max(0, p - q) after a rejection (step 4) or p for the bonus token
// (step 5), sums it per 512-logit tile and per 8192-logit segment, and the last
// workgroup of the row walks segment sums, tile sums and one tile to the inverse-CDF
// token.  All workgroups of a row run on one XCD so that final tile re-read hits
// that XCD's L2.
#include <float.h>
#include <limits.h>

#include "sv_internal.h"

namespace sv {

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
        int64_t vt = in ? (int64_t)g + 1 : 0, vd = in ? (int64_t)g : 0;
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
            // vector slots of row i: target positions then draft positions
            const int64_t s0 = t_off + d_off;
            if (s0 < P.nvec) {
                int64_t n = 2 * (int64_t)g + 1;
                if (n > P.nvec - s0) n = P.nvec - s0;
                for (int64_t k = 0; k < n; ++k) P.vec_row[s0 + k] = (int32_t)i;
            }
        }
        __syncthreads();
        if (tid == 1023) { carry_t = pt + it; carry_d = pd + id; }
        __syncthreads();
    }
    if (tid == 0) P.hdr->status = (bad || carry_t != P.nT) ? ST_BAD_GAMMA : 0;
}

// ===========================================================================
// pass 1: per-vector statistics
// ===========================================================================
struct SampleState {
    float m;        // running maximum
    float mref;     // logit the reference exponent was taken at (-inf: none yet)
    float Mref;     // fp32(mref * c_hi)
    bool fast;      // |Mref| < 2^30: single-fma argument against Mref
    bool nan_seen;  // a NaN arrived while no finite logit had been seen
    double R;       // s holds sum 2^(z c - R)
    double s;
};

template <int N>
__device__ __forceinline__ void sample_chunk(SampleState &st, const float *x, const TempConst &tc)
{
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) cm = fmaxf(cm, x[i]);
    st.m = fmaxf(st.m, cm);
    // new reference only when the maximum first appears or climbs by 16 binades,
    // so exponents stay <= 16 without a rescale per chunk
    if (cm > st.mref && (st.mref == -INFINITY || (cm - st.mref) * tc.c_hi > 16.0f)) {
        const float M = cm * tc.c_hi;
        const bool fast = fabsf(M) < kFastRef;
        const double R = fast ? (double)M : (double)cm * tc.c_eff;
        if (st.mref != -INFINITY) st.s *= exp2(st.R - R);
        st.mref = cm;
        st.Mref = M;
        st.fast = fast;
        st.R = R;
    }
    if (st.mref == -INFINITY) {
#pragma unroll
        for (int i = 0; i < N; ++i) st.nan_seen |= (x[i] != x[i]);
        return;
    }
    float e[N];
    if (st.fast) {
#pragma unroll
        for (int i = 0; i < N; ++i) e[i] = fast_exp2(fmaf(x[i], tc.c_lo, fmaf(x[i], tc.c_hi, -st.Mref)));
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float d = x[i] - st.mref;
            e[i] = fast_exp2(fmaf(d, tc.c_hi, d * tc.c_lo));
        }
    }
#pragma unroll
    for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
    st.s += (double)e[0];
}

struct GreedyState {
    float best;
    int32_t idx;
    bool nan_seen;
};

template <int DT, bool AL, bool GREEDY>
__device__ __forceinline__ Partial reduce_segment(const void *base, int64_t u0, int64_t u1, int64_t V,
                                                  const TempConst &tc)
{
    constexpr int N = kUnroll * kUnitElems;
    __shared__ float sh_f[kWaves];
    __shared__ double sh_d[kWaves];
    __shared__ int sh_i[kWaves], sh_n[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    SampleState st{-INFINITY, -INFINITY, 0.0f, false, false, 0.0, 0.0};
    GreedyState gs{-INFINITY, INT32_MAX, false};

    for (int64_t ub = u0 + tid; ub < u1; ub += (int64_t)kBlock * kUnroll) {
        float x[N];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t u = ub + (int64_t)k * kBlock;
            if (u < u1) {
                load_unit<DT, AL>(base, u, V, x + k * kUnitElems);
            } else {
#pragma unroll
                for (int e = 0; e < kUnitElems; ++e) x[k * kUnitElems + e] = -INFINITY;
            }
        }
        if constexpr (GREEDY) {
            float cm = x[0];
#pragma unroll
            for (int i = 1; i < N; ++i) cm = fmaxf(cm, x[i]);
            bool nan = false;
#pragma unroll
            for (int i = 0; i < N; ++i) nan |= (x[i] != x[i]);
            gs.nan_seen |= nan;
            if (cm > gs.best) {
                gs.best = cm;
#pragma unroll
                for (int i = N - 1; i >= 0; --i)
                    if (x[i] == cm)
                        gs.idx = (int32_t)((ub + (int64_t)(i / kUnitElems) * kBlock) * kUnitElems +
                                           (i % kUnitElems));
            }
        } else {
            sample_chunk<N>(st, x, tc);
        }
    }

    Partial out;
    if constexpr (GREEDY) {
        float b = wave_max(gs.best);
        if (lane == 0) sh_f[wave] = b;
        __syncthreads();
        b = sh_f[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) b = fmaxf(b, sh_f[w]);
        int cand = (gs.best == b) ? gs.idx : INT32_MAX;
        cand = wave_min_int(cand);
        int nan = wave_or_int(gs.nan_seen ? 1 : 0);
        if (lane == 0) { sh_i[wave] = cand; sh_n[wave] = nan; }
        __syncthreads();
        int idx = sh_i[0];
        int anynan = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { idx = min(idx, sh_i[w]); anynan |= sh_n[w]; }
        out.m = b;
        out.idx = idx;
        out.s = anynan ? __longlong_as_double(0x7ff8000000000000LL) : 0.0;
    } else {
        // this thread's sum relative to its own maximum
        double s_m;
        if (st.mref == -INFINITY)
            s_m = 0.0;
        else
            s_m = st.s * exp2(st.R - (double)st.m * tc.c_eff);
        if (st.nan_seen) s_m = __longlong_as_double(0x7ff8000000000000LL);
        float mw = wave_max(st.m);
        if (lane == 0) sh_f[wave] = mw;
        __syncthreads();
        mw = sh_f[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mw = fmaxf(mw, sh_f[w]);
        double c = (st.m == -INFINITY) ? s_m : s_m * exp2(((double)st.m - (double)mw) * tc.c_eff);
        c = wave_sum(c);
        if (lane == 0) sh_d[wave] = c;
        __syncthreads();
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sh_d[w];
        out.m = mw;
        out.idx = 0;
        out.s = s;
    }
    return out;
}

template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void stats_kernel(Params P)
{
    const int64_t item = blockIdx.x;
    const int64_t slot = item / P.geo.nseg;
    const int32_t seg = (int32_t)(item - slot * P.geo.nseg);
    int32_t row;
    RowGeom G;
    if (P.gamma != nullptr) {
        if (P.hdr->status != 0) return;
        row = P.vec_row[slot];
        G = row_geom(P, row);
    } else {
        const int64_t per = 2 * (int64_t)P.gamma_uniform + 1;
        row = (int32_t)(slot / per);
        G = row_geom(P, row);
    }
    const int64_t k = slot - (G.t_off + G.d_off);
    const bool is_target = k <= G.gamma;
    const float T = P.temperature[row];
    const int32_t rm = row_mode(P.mode, T);
    if (rm == ROW_BAD_TEMP) return;
    if (rm == ROW_GREEDY && !is_target) return;
    const int64_t vrow = is_target ? G.t_off + k : G.d_off + (k - G.gamma - 1);
    const void *base = vec_ptr(is_target ? P.target : P.draft, DT, vrow, P.V);
    const int64_t u0 = (int64_t)seg * P.geo.seg_units;
    int64_t u1 = u0 + P.geo.seg_units;
    if (u1 > P.geo.nunits) u1 = P.geo.nunits;
    Partial out;
    if (rm == ROW_GREEDY) {
        TempConst tc{1.0f, 0.0f, 1.0};
        out = reduce_segment<DT, AL, true>(base, u0, u1, P.V, tc);
    } else {
        const TempConst tc = temp_const(T);
        out = reduce_segment<DT, AL, false>(base, u0, u1, P.V, tc);
    }
    if (threadIdx.x == 0) P.parts[slot * P.geo.nseg + seg] = out;
}

// ===========================================================================
// accept scan: one wave per row
// ===========================================================================
__device__ __forceinline__ void combine_sample(const Params &P, int64_t slot, const TempConst &tc,
                                               float &m, double &S)
{
    const Partial *pp = P.parts + slot * P.geo.nseg;
    m = -INFINITY;
    for (int s = 0; s < P.geo.nseg; ++s) m = fmaxf(m, pp[s].m);
    S = 0.0;
    for (int s = 0; s < P.geo.nseg; ++s) {
        const Partial q = pp[s];
        S += (q.m == -INFINITY) ? q.s : q.s * exp2(((double)q.m - (double)m) * tc.c_eff);
    }
}

__device__ __forceinline__ void combine_greedy(const Params &P, int64_t slot, float &val, int32_t &idx,
                                               bool &nan)
{
    const Partial *pp = P.parts + slot * P.geo.nseg;
    val = -INFINITY;
    for (int s = 0; s < P.geo.nseg; ++s) val = fmaxf(val, pp[s].m);
    idx = INT32_MAX;
    nan = false;
    for (int s = 0; s < P.geo.nseg; ++s) {
        const Partial q = pp[s];
        if (q.m == val && q.idx < idx) idx = q.idx;
        nan |= (q.s != q.s);
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void scan_kernel(Params P)
{
    const int lane = threadIdx.x & 63;
    const int32_t row = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const double qnan = __longlong_as_double(0x7ff8000000000000LL);

    if (P.gamma != nullptr && P.hdr->status != 0) {
        // inconsistent gamma array: every row and slot is invalid
        const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
        const int64_t nthreads = (int64_t)gridDim.x * kBlock;
        for (int64_t s = gid; s < P.nT; s += nthreads) P.emitted[s] = -1;
        for (int64_t s = gid; s < P.nD; s += nthreads) {
            if (P.p_x) P.p_x[s] = qnan;
            if (P.q_x) P.q_x[s] = qnan;
        }
        if (row < P.B && lane == 0) {
            P.n_accepted[row] = -1;
            if (P.row_status) P.row_status[row] = ST_BAD_GAMMA;
            if (P.resid) P.resid[row] = qnan;
            P.draws[row].kind = DRAW_NONE;
            P.counters[row] = 0;
        }
        return;
    }
    if (row >= P.B) return;
    if (lane == 0) P.counters[row] = 0;

    const RowGeom G = row_geom(P, row);
    const int32_t g = G.gamma;
    const int64_t slot0 = G.t_off + G.d_off;
    const float T = P.temperature[row];
    const int32_t rm = row_mode(P.mode, T);
    const bool greedy = rm == ROW_GREEDY;
    const TempConst tc = temp_const(rm == ROW_SAMPLE ? T : 1.0f);
    const double Td = (double)T;
    int status = (rm == ROW_BAD_TEMP) ? ST_BAD_TEMP : 0;
    int32_t K = g;
    bool found = false;

    if (rm != ROW_BAD_TEMP) {
        for (int base = 0; base <= g; base += 64) {
            const int j = base + lane;
            bool reject = false;
            if (j <= g) {
                const int64_t ts = slot0 + j;
                int32_t x = 0;
                bool x_ok = false;
                if (j < g) {
                    x = P.tokens[G.d_off + j];
                    x_ok = x >= 0 && (int64_t)x < P.V;
                    if (!x_ok) status |= ST_BAD_TOKEN;
                }
                if (greedy) {
                    float val;
                    int32_t idx;
                    bool nan;
                    combine_greedy(P, ts, val, idx, nan);
                    if (nan || !(val > -INFINITY && val < INFINITY)) status |= ST_NONFINITE;
                    if (j < g) reject = x != idx;
                } else {
                    float mt;
                    double St;
                    combine_sample(P, ts, tc, mt, St);
                    if (!(St > 0.0 && St < INFINITY)) status |= ST_NONFINITE;
                    if (j < g) {
                        float md;
                        double Sd;
                        combine_sample(P, slot0 + g + 1 + j, tc, md, Sd);
                        if (!(Sd > 0.0 && Sd < INFINITY)) status |= ST_NONFINITE;
                        double px = qnan, qx = qnan;
                        if (x_ok && St > 0.0 && St < INFINITY && Sd > 0.0 && Sd < INFINITY) {
                            const float zt = load_logit<DT>(vec_ptr(P.target, DT, G.t_off + j, P.V), x);
                            const float zd = load_logit<DT>(vec_ptr(P.draft, DT, G.d_off + j, P.V), x);
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
                            reject = !((double)P.uniforms[G.t_off + j] < ratio);
                        }
                        if (P.p_x) P.p_x[G.d_off + j] = px;
                        if (P.q_x) P.q_x[G.d_off + j] = qx;
                    }
                }
            }
            const unsigned long long rb = __ballot(reject);
            if (!found && rb != 0ull) {
                K = base + __ffsll((long long)rb) - 1;
                found = true;
            }
        }
    }
    status = wave_or_int(status);
    const bool invalid = (status & ST_INVALID) != 0;

    // emitted tokens, -1 past the drawn position
    int32_t aK = -1;
    if (!invalid && greedy && lane == 0) {
        float val;
        bool nan;
        combine_greedy(P, slot0 + K, val, aK, nan);
    }
    aK = __shfl(aK, 0);
    for (int j = lane; j <= g; j += 64) {
        int32_t e = -1;
        if (!invalid) {
            if (j < K) e = P.tokens[G.d_off + j];
            else if (j == K && greedy) e = aK;
        }
        P.emitted[G.t_off + j] = e;
        if (j < g && (invalid || greedy)) {
            if (P.p_x) P.p_x[G.d_off + j] = qnan;
            if (P.q_x) P.q_x[G.d_off + j] = qnan;
        }
    }
    if (lane == 0) {
        P.n_accepted[row] = invalid ? -1 : K;
        if (P.row_status) P.row_status[row] = status;
        RowDraw D{};
        D.kind = DRAW_NONE;
        if (!invalid && !greedy) {
            D.kind = K < g ? DRAW_RESIDUAL : DRAW_BONUS;
            D.K = K;
            D.t_row = (int32_t)(G.t_off + K);
            D.d_row = (int32_t)(G.d_off + K);
            D.u = P.uniforms[G.t_off + g];
            D.t_slot = (int32_t)(G.t_off + K);
            combine_sample(P, slot0 + K, tc, D.m_t, D.S_t);
            if (K < g) combine_sample(P, slot0 + g + 1 + K, tc, D.m_d, D.S_d);
        } else if (P.resid) {
            P.resid[row] = qnan;
        }
        P.draws[row] = D;
    }
}

// ===========================================================================
// pass 2: residual / bonus weights and the inverse-CDF draw
// ===========================================================================
struct DrawConst {
    TempConst tc;
    float Mt, Md, mt, md;
    float Ft, Fd;           // unnormalized -> probability
    bool fast_t, fast_d;
    bool residual;
};

__device__ __forceinline__ DrawConst draw_const(const RowDraw &D, float T)
{
    DrawConst c;
    c.tc = temp_const(T);
    c.residual = D.kind == DRAW_RESIDUAL;
    c.mt = D.m_t;
    c.Mt = D.m_t * c.tc.c_hi;
    c.fast_t = fabsf(c.Mt) < kFastRef;
    c.Ft = c.fast_t ? (float)(exp2((double)c.Mt - (double)D.m_t * c.tc.c_eff) / D.S_t)
                    : (float)(1.0 / D.S_t);
    c.md = D.m_d;
    c.Md = D.m_d * c.tc.c_hi;
    c.fast_d = fabsf(c.Md) < kFastRef;
    c.Fd = 0.0f;
    if (c.residual)
        c.Fd = c.fast_d ? (float)(exp2((double)c.Md - (double)D.m_d * c.tc.c_eff) / D.S_d)
                        : (float)(1.0 / D.S_d);
    return c;
}

__device__ __forceinline__ float unnorm(float z, float M, float m, bool fast, const TempConst &tc)
{
    if (fast) return fast_exp2(fmaf(z, tc.c_lo, fmaf(z, tc.c_hi, -M)));
    const float d = z - m;
    return fast_exp2(fmaf(d, tc.c_hi, d * tc.c_lo));
}

// weights w (residual or p) and target probabilities p of one unit
template <int DT, bool AL>
__device__ __forceinline__ void unit_weights(const DrawConst &c, const void *tb, const void *db, int64_t unit,
                                             int64_t V, float *w, float *p)
{
    float zt[kUnitElems];
    load_unit<DT, AL>(tb, unit, V, zt);
#pragma unroll
    for (int e = 0; e < kUnitElems; ++e) p[e] = unnorm(zt[e], c.Mt, c.mt, c.fast_t, c.tc) * c.Ft;
    if (c.residual) {
        float zd[kUnitElems];
        load_unit<DT, AL>(db, unit, V, zd);
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const float q = unnorm(zd[e], c.Md, c.md, c.fast_d, c.tc) * c.Fd;
            w[e] = fmaxf(0.0f, p[e] - q);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) w[e] = p[e];
    }
}

// Within the `n` sums at arr (stride 2 doubles, field 0 = w, 1 = p), with `carry`
// already accumulated before them, find the first index whose running sum exceeds
// t; if none, the last index with a positive value.  Returns the index and the
// running sum before it.  Executed by one full wave.
__device__ __forceinline__ int find_in_sums(const Sum2 *arr, int n, bool use_p, double t, double carry,
                                            int lane, double &before)
{
    int found = -1, last_pos = -1;
    double before_found = 0.0, before_last = 0.0;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int i = c0 + lane;
        const double v = i < n ? (use_p ? arr[i].p : arr[i].w) : 0.0;
        const double incl = wave_inclusive_sum(v, lane) + carry;
        const unsigned long long hit = __ballot(i < n && incl > t);
        const unsigned long long pos = __ballot(i < n && v > 0.0);
        if (pos) {
            const int l = 63 - __clzll((long long)pos);
            last_pos = c0 + l;
            before_last = __shfl(incl - v, l);
        }
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            found = c0 + l;
            before_found = __shfl(incl - v, l);
            break;
        }
        carry = __shfl(incl, 63);
    }
    if (found >= 0) {
        before = before_found;
        return found;
    }
    before = before_last;
    return last_pos;
}

__device__ __forceinline__ double sum_all(const Sum2 *arr, int n, bool use_p, int lane)
{
    double carry = 0.0;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int i = c0 + lane;
        const double v = i < n ? (use_p ? arr[i].p : arr[i].w) : 0.0;
        const double incl = wave_inclusive_sum(v, lane) + carry;
        carry = __shfl(incl, 63);
    }
    return carry;
}

template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void draw_kernel(Params P)
{
    __shared__ double sh_w[kWaves], sh_p[kWaves];
    __shared__ int sh_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // all segments of a row on one XCD: workgroup w runs on XCD w % 8
    const int64_t wg = blockIdx.x;
    const int32_t xcd = (int32_t)(wg % kXcds);
    const int64_t local = wg / kXcds;
    const int64_t rk = local / P.geo.nseg2;
    const int32_t seg = (int32_t)(local - rk * P.geo.nseg2);
    const int64_t row64 = (int64_t)xcd + (int64_t)kXcds * rk;
    if (row64 >= P.B) return;
    const int32_t row = (int32_t)row64;
    const RowDraw D = P.draws[row];
    if (D.kind == DRAW_NONE) return;

    const DrawConst c = draw_const(D, P.temperature[row]);
    const void *tb = vec_ptr(P.target, DT, D.t_row, P.V);
    const void *db = c.residual ? vec_ptr(P.draft, DT, D.d_row, P.V) : nullptr;
    Sum2 *tiles = P.tiles + (int64_t)row * P.geo.ntiles;
    Sum2 *segs = P.segs + (int64_t)row * P.geo.nseg2;

    // ---- tile and segment sums ----
    const int64_t t0 = (int64_t)seg * kTilesPerSeg;
    int64_t t1 = t0 + kTilesPerSeg;
    if (t1 > P.geo.ntiles) t1 = P.geo.ntiles;
    double acc_w = 0.0, acc_p = 0.0;
    for (int64_t tile = t0 + wave; tile < t1; tile += kWaves) {
        const int64_t unit = tile * kTileUnits + lane;
        float w[kUnitElems], p[kUnitElems];
        float lw = 0.0f, lp = 0.0f;
        if (unit < P.geo.nunits) {
            unit_weights<DT, AL>(c, tb, db, unit, P.V, w, p);
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) { lw += w[e]; lp += p[e]; }
        }
        const double tw = wave_sum((double)lw), tp = wave_sum((double)lp);
        if (lane == 0) tiles[tile] = Sum2{tw, tp};
        acc_w += tw;
        acc_p += tp;
    }
    if (lane == 0) { sh_w[wave] = acc_w; sh_p[wave] = acc_p; }
    __syncthreads();
    if (tid == 0) {
        double sw = 0.0, sp = 0.0;
        for (int w = 0; w < kWaves; ++w) { sw += sh_w[w]; sp += sh_p[w]; }
        segs[seg] = Sum2{sw, sp};
        __threadfence();
        const int old = atomicAdd(&P.counters[row], 1);
        sh_last = (old == P.geo.nseg2 - 1);
    }
    __syncthreads();
    if (!sh_last || wave != 0) return;
    __threadfence();

    // ---- the last workgroup of the row: inverse CDF ----
    const int nseg2 = P.geo.nseg2;
    bool use_p = false;
    double W = sum_all(segs, nseg2, false, lane);
    if (c.residual && !(W > 0.0)) {
        use_p = true;
        W = sum_all(segs, nseg2, true, lane);
    }
    const double t = (double)D.u * W;
    double before;
    const int g = find_in_sums(segs, nseg2, use_p, t, 0.0, lane, before);
    int32_t token = -1;
    if (g >= 0) {
        const int64_t gt0 = (int64_t)g * kTilesPerSeg;
        int nt = kTilesPerSeg;
        if (gt0 + nt > P.geo.ntiles) nt = (int)(P.geo.ntiles - gt0);
        double before_tile;
        const int tl = find_in_sums(tiles + gt0, nt, use_p, t, before, lane, before_tile);
        if (tl >= 0) {
            const int64_t tile = gt0 + tl;
            const int64_t unit = tile * kTileUnits + lane;
            float w[kUnitElems], p[kUnitElems];
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) w[e] = p[e] = 0.0f;
            if (unit < P.geo.nunits) unit_weights<DT, AL>(c, tb, db, unit, P.V, w, p);
            double lsum = 0.0;
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) lsum += (double)(use_p ? p[e] : w[e]);
            const double incl = wave_inclusive_sum(lsum, lane);
            double cum = before_tile + incl - lsum;
            int cand = -1, lastpos = -1;
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e) {
                const float we = use_p ? p[e] : w[e];
                cum += (double)we;
                if (cand < 0 && cum > t) cand = e;
                if (we > 0.0f) lastpos = e;
            }
            const unsigned long long hit = __ballot(cand >= 0);
            if (hit) {
                const int l = __ffsll((long long)hit) - 1;
                token = (int32_t)(__shfl((int)(unit * kUnitElems) + cand, l));
            } else {
                const unsigned long long pos = __ballot(lastpos >= 0);
                if (pos) {
                    const int l = 63 - __clzll((long long)pos);
                    token = (int32_t)(__shfl((int)(unit * kUnitElems) + lastpos, l));
                }
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

hipError_t launch_prepare(const Params &P, hipStream_t s)
{
    return launch((const void *)prepare_kernel, 1, 1024, P, s);
}

hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const int64_t blocks = P.nvec * P.geo.nseg;
    const void *fn = dtype == 0 ? (aligned ? (const void *)stats_kernel<0, true> : (const void *)stats_kernel<0, false>)
                                : (aligned ? (const void *)stats_kernel<1, true> : (const void *)stats_kernel<1, false>);
    return launch(fn, blocks, kBlock, P, s);
}

hipError_t launch_scan(const Params &P, hipStream_t s, int dtype)
{
    const int64_t blocks = ((int64_t)P.B + kWaves - 1) / kWaves;
    const void *fn = dtype == 0 ? (const void *)scan_kernel<0> : (const void *)scan_kernel<1>;
    return launch(fn, blocks, kBlock, P, s);
}

hipError_t launch_draw(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const int64_t rows8 = ((int64_t)P.B + kXcds - 1) / kXcds;
    const int64_t blocks = rows8 * kXcds * P.geo.nseg2;
    const void *fn = dtype == 0 ? (aligned ? (const void *)draw_kernel<0, true> : (const void *)draw_kernel<0, false>)
                                : (aligned ? (const void *)draw_kernel<1, true> : (const void *)draw_kernel<1, false>);
    return launch(fn, blocks, kBlock, P, s);
}

}  // namespace sv
