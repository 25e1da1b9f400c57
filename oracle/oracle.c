/*
 * fp64 CPU oracle of the speculative-sampling verification step.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load this file's library.  The product library never links, loads
 * or calls it, and it shares no code, header or table with the HIP path.
 *
 * It computes, plainly and in float64, what one verification round computes:
 *
 *  - temperature softmax of every position's logits, y_i = exp(z_i/t) / sum_j exp(z_j/t)
 *    (brunomaga.github.io "inference-distillation-speculative-decoding", section
 *    "Knowledge distillation", the softened-output equation), with the same t for the
 *    target distribution p and the drafter distribution q (rayaq.ca "Speculative
 *    decoding", section "Why the output is exactly the target's", last paragraph);
 *    evaluated with the maximum logit subtracted first, which leaves y unchanged;
 *  - the left-to-right accept test: draft x_j is kept iff u_j < min(1, p_j(x_j)/q_j(x_j)),
 *    stopping at the first rejection (rayaq.ca "Speculative decoding", section
 *    "One round", step 3);
 *  - on a rejection at position K, one draw from the residual
 *    r = max(0, p_K - q_K) / sum max(0, p_K - q_K) (same section, step 4);
 *  - if all drafts are kept, one bonus draw from p at the position after the last
 *    draft (same section, step 5);
 *  - the greedy variant: keep drafts while they equal the target's argmax, then emit
 *    the target's argmax at the first mismatch or after the last draft (rayaq.ca
 *    "Speculative decoding", section "The greedy case"; brunomaga.github.io, section
 *    "Draft-model speculative decoding", greedy paragraph).
 *
 * Readings where the pages leave a step open:
 *  - p is the target, q the drafter (the rayaq.ca and cgnarendiran.github.io naming;
 *    brunomaga.github.io swaps the letters, not the rule);
 *  - the test is strict, u < ratio, with u in [0, 1);
 *  - uniforms are inputs: slot j < gamma drives accept test j, slot gamma drives the
 *    single categorical draw (residual or bonus);
 *  - a categorical draw is the inverse CDF in token order: with weights w,
 *    W = sum(w), t = u * W, the token is the smallest v whose running sum exceeds t;
 *  - q(x) = 0 gives ratio 1 if p(x) > 0, else 0 (flagged Q_ZERO);
 *  - residual mass W = 0 at a rejection (possible only through rounding) falls back to
 *    drawing from p_K (flagged ZERO_RESID);
 *  - temperature t <= 0 in sampling mode makes that row greedy (the t -> 0 limit);
 *  - greedy argmax is taken on the raw logits, lowest index on ties;
 *  - a NaN or +inf logit, or a position whose logits are all -inf, makes the row
 *    invalid (NONFINITE); -inf elsewhere is an ordinary zero-probability token;
 *  - a decision whose threshold is within eps of its input (|u - ratio| < eps for a
 *    test, |C - t| < eps * W at an interior edge of the drawn token's CDF interval
 *    for a draw; eps = 1e-5 unless the caller passes another) is "near": flag_pos
 *    holds a row's first near decision, flags[] marks every one (slot t_off + j for
 *    test j, slot t_off + gamma for the draw), and [draw_lo, draw_hi] bound the tokens
 *    a near draw could return (those whose CDF interval comes within eps * W of the
 *    threshold), so that a comparison with arithmetic of another precision can hold
 *    each decision to exactly what its input fixes.
 */
#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------- */
/* element access: exact upcast of bf16 / fp32 / fp64 logits to double       */
/* ------------------------------------------------------------------------- */
static double logit_at(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    return ((const double *)base)[idx];
}

static const void *vector_ptr(const void *base, int dtype, int64_t row, int64_t V)
{
    size_t esz = dtype == ORACLE_BF16 ? 2 : dtype == ORACLE_F32 ? 4 : 8;
    return (const char *)base + (size_t)row * (size_t)V * esz;
}

/* ------------------------------------------------------------------------- */
/* temperature softmax of one position                                        */
/* ------------------------------------------------------------------------- */

/* NaN or +inf anywhere, or every element -inf: the position has no softmax. */
static int vector_nonfinite(const void *z, int dtype, int64_t V)
{
    int any_above_neg_inf = 0;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(z, dtype, v);
        if (isnan(x) || x == INFINITY)
            return 1;
        if (x != -INFINITY)
            any_above_neg_inf = 1;
    }
    return !any_above_neg_inf;
}

/* m = max z, S = sum_v exp((z_v - m)/T), summed in index order. */
/* The logit of token v after filtering at theta: tokens below it drop out (their
 * probability is 0, as for a logit of -inf). */
static double kept_logit(const void *z, int dtype, int64_t v, double theta)
{
    const double x = logit_at(z, dtype, v);
    return x >= theta ? x : -INFINITY;
}

/* m = max z, S = sum_v exp((z_v - m)/T) over the tokens kept at theta, in index order. */
static void vector_max_sumexp(const void *z, int dtype, int64_t V, double T, double theta,
                              double *m_out, double *S_out)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(z, dtype, v);
        if (x > m)
            m = x;
    }
    double S = 0.0;
    for (int64_t v = 0; v < V; ++v)
        S += exp((kept_logit(z, dtype, v, theta) - m) / T);
    *m_out = m;
    *S_out = S;
}

static int softmax_kept(const void *z, int dtype, int64_t V, double T, double theta, double *p)
{
    if (!z || !p || V <= 0 || !(T > 0) || !isfinite(T))
        return -1;
    if (vector_nonfinite(z, dtype, V))
        return ORACLE_NONFINITE;
    double m, S;
    vector_max_sumexp(z, dtype, V, T, theta, &m, &S);
    for (int64_t v = 0; v < V; ++v)
        p[v] = exp((kept_logit(z, dtype, v, theta) - m) / T) / S;
    return 0;
}

int oracle_softmax(const void *z, int dtype, int64_t V, double T, double *p)
{
    return softmax_kept(z, dtype, V, T, -INFINITY, p);
}

/* ------------------------------------------------------------------------- */
/* top-k and top-p filtering                                                   */
/* ------------------------------------------------------------------------- */
static int cmp_desc(const void *a, const void *b)
{
    const double x = *(const double *)a, y = *(const double *)b;
    return x > y ? -1 : (x < y ? 1 : 0);
}

/* The logit threshold theta of a filtered distribution: a token is kept iff its logit
 * is >= theta (-inf: no filtering).  The pages require any such filter to be applied
 * to both p and q before the test (rayaq.ca "Speculative decoding", section "Why the
 * output is exactly the target's", last paragraph; section "Tradeoffs").
 *  - top-k (0 < top_k < V): theta_k = the top_k-th largest logit, counted with
 *    multiplicity; every token tied with it is kept too;
 *  - top-p (0 < top_p < 1), on the distribution left by top-k: tokens are taken in
 *    decreasing logit order, a whole group of equal logits at a time, until their
 *    probability reaches top_p; theta_p = the logit of the last group taken;
 *  - theta = max(theta_k, theta_p).
 * *near = 1 when top_p lies within eps of the cumulative probability on either side
 * of the last group's step. */
int oracle_filter_threshold(const void *z, int dtype, int64_t V, double T, int64_t top_k, double top_p,
                            double eps, double *theta_out, int *near)
{
    *theta_out = -INFINITY;
    if (near)
        *near = 0;
    if (!z || V <= 0 || !(T > 0) || !isfinite(T))
        return -1;
    const int use_k = top_k > 0 && top_k < V;
    const int use_p = top_p > 0 && top_p < 1;
    if ((!use_k && !use_p) || vector_nonfinite(z, dtype, V))
        return 0;
    double *s = malloc(sizeof(double) * (size_t)V);
    if (!s)
        return -1;
    for (int64_t v = 0; v < V; ++v)
        s[v] = logit_at(z, dtype, v);
    qsort(s, (size_t)V, sizeof(double), cmp_desc);
    double theta = use_k ? s[top_k - 1] : -INFINITY;
    if (use_p) {
        const double m = s[0];
        double S = 0.0;
        for (int64_t i = 0; i < V && s[i] >= theta; ++i)
            S += exp((s[i] - m) / T);
        const double target = top_p * S;
        double cum = 0.0;
        for (int64_t i = 0; i < V && s[i] >= theta;) {
            const double val = s[i];
            const double before = cum;
            for (; i < V && s[i] == val; ++i)
                cum += exp((s[i] - m) / T);
            if (cum >= target) {
                if (near)
                    *near = (cum - target < eps * S) || (target - before < eps * S);
                theta = val;
                break;
            }
        }
    }
    free(s);
    *theta_out = theta;
    return 0;
}

/* first index of the maximum of the raw logits */
int64_t oracle_argmax(const void *z, int dtype, int64_t V)
{
    int64_t best = 0;
    double bv = logit_at(z, dtype, 0);
    for (int64_t v = 1; v < V; ++v) {
        double x = logit_at(z, dtype, v);
        if (x > bv) {
            bv = x;
            best = v;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------- */
/* one position: alpha, residual mass and residual distribution               */
/* ------------------------------------------------------------------------- */
int oracle_position(const void *zt, const void *zd, int dtype, int64_t V, double T, double *p,
                    double *q, double *alpha, double *resid_mass, double *residual)
{
    double *pp = p ? p : malloc(sizeof(double) * (size_t)V);
    double *qq = q ? q : malloc(sizeof(double) * (size_t)V);
    int rc = 0;
    if (!pp || !qq) {
        rc = -1;
        goto out;
    }
    rc = oracle_softmax(zt, dtype, V, T, pp);
    if (rc == 0)
        rc = oracle_softmax(zd, dtype, V, T, qq);
    if (rc != 0)
        goto out;
    double a = 0.0, w = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        a += fmin(pp[v], qq[v]);
        w += fmax(0.0, pp[v] - qq[v]);
    }
    if (alpha)
        *alpha = a;
    if (resid_mass)
        *resid_mass = w;
    if (residual)
        for (int64_t v = 0; v < V; ++v)
            residual[v] = w > 0 ? fmax(0.0, pp[v] - qq[v]) / w : 0.0;
out:
    if (!p)
        free(pp);
    if (!q)
        free(qq);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* the inverse-CDF draw                                                        */
/* ------------------------------------------------------------------------- */
/* The draw with weights w: W = sum(w), t = u * W, the token is the smallest v whose
 * running sum C_v exceeds t.  *near_edge = 1 when t lies within eps * W of an interior
 * edge of that token's interval [C_{v-1}, C_v); then [*lo, *hi] are the first and last
 * tokens with positive weight whose interval comes within eps * W of t (the tokens a
 * draw could return whose threshold or running sums were off by eps * W).  Otherwise
 * *lo = *hi = the token. */
int64_t oracle_inverse_cdf_range(const double *w, int64_t V, double u, double eps, double *W_out,
                                 int *near_edge, int64_t *lo, int64_t *hi)
{
    double W = 0.0;
    for (int64_t v = 0; v < V; ++v)
        W += w[v];
    double t = u * W;
    double C = 0.0, C_prev = 0.0;
    int64_t token = -1;
    for (int64_t v = 0; v < V; ++v) {
        C_prev = C;
        C += w[v];
        if (C > t) {
            token = v;
            break;
        }
    }
    if (token < 0) { /* only through rounding: the last token with positive weight */
        for (int64_t v = V - 1; v >= 0; --v)
            if (w[v] > 0) {
                token = v;
                break;
            }
        C = W;
        C_prev = W - (token >= 0 ? w[token] : 0.0);
    }
    /* only interior edges are decision boundaries: the lower edge when some earlier
       token has weight, the upper edge when some later token has weight */
    const int near = (C_prev > 0 && fabs(C_prev - t) < eps * W) || (C < W && fabs(C - t) < eps * W);
    int64_t a = token, b = token;
    if (near) {
        double c = 0.0;
        a = b = -1;
        for (int64_t v = 0; v < V; ++v) {
            const double before = c;
            c += w[v];
            if (w[v] > 0 && c >= t - eps * W && before <= t + eps * W) {
                if (a < 0)
                    a = v;
                b = v;
            }
        }
        if (a < 0)
            a = b = token;
    }
    if (near_edge)
        *near_edge = near;
    if (lo)
        *lo = a;
    if (hi)
        *hi = b;
    if (W_out)
        *W_out = W;
    return token;
}

int64_t oracle_inverse_cdf(const double *w, int64_t V, double u, double eps, double *W_out,
                           int *near_edge)
{
    return oracle_inverse_cdf_range(w, V, u, eps, W_out, near_edge, NULL, NULL);
}

/* ------------------------------------------------------------------------- */
/* the verification round, one batch                                           */
/* ------------------------------------------------------------------------- */
/* Cache entries to keep after a round that kept K drafts over a prefix of n: the
 * prefix, the last token and the kept drafts (rayaq.ca "Speculative decoding",
 * section "Verification attention and the cache"). */
static int32_t kept_cache_entries(const int32_t *cache_len, int32_t i, int K)
{
    const int32_t n = cache_len ? cache_len[i] : 0;
    return n + K + 1;
}

/* The acceptance probability min(1, p(x)/q(x)) of draft token x at one position
 * (rayaq.ca "Speculative decoding", section "One round", step 3), with p(x) and q(x)
 * from the temperature softmax of the tokens kept at theta_t and theta_d; q(x) = 0
 * gives 1 if p(x) > 0, else 0 (*q_zero = 1). */
static double accept_ratio(const void *zt, const void *zd, int dtype, int64_t V, double T, int64_t x,
                           double theta_t, double theta_d, double *px_out, double *qx_out, int *q_zero)
{
    double mt, St, md, Sd;
    vector_max_sumexp(zt, dtype, V, T, theta_t, &mt, &St);
    vector_max_sumexp(zd, dtype, V, T, theta_d, &md, &Sd);
    double px = exp((kept_logit(zt, dtype, x, theta_t) - mt) / T) / St;
    double qx = exp((kept_logit(zd, dtype, x, theta_d) - md) / T) / Sd;
    *px_out = px;
    *qx_out = qx;
    *q_zero = 0;
    double ratio;
    if (qx > 0) {
        ratio = px / qx;
        if (ratio > 1.0)
            ratio = 1.0;
    } else {
        ratio = px > 0 ? 1.0 : 0.0;
        *q_zero = 1;
    }
    return ratio;
}

static void invalidate_row(int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                           double *resid, int64_t i, int64_t t0, int64_t d0, int g)
{
    n_accepted[i] = -1;
    for (int j = 0; j <= g; ++j)
        emitted[t0 + j] = -1;
    if (p_x)
        for (int j = 0; j < g; ++j)
            p_x[d0 + j] = NAN;
    if (q_x)
        for (int j = 0; j < g; ++j)
            q_x[d0 + j] = NAN;
    if (resid)
        resid[i] = NAN;
}

int oracle_verify(const void *target, const void *draft, int dtype, int64_t V, int32_t B,
                  int64_t n_target_rows, const int32_t *draft_tokens, const float *uniforms,
                  const float *temperature, const int32_t *gamma_per_row, int mode,
                  int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                  double *resid_mass, int32_t *row_status, int32_t *flag_pos, double flag_eps,
                  int nthreads);

/* The round with early exit: positions are read left to right and nothing after the
 * first rejection is read (rayaq.ca "Speculative decoding", section "One round",
 * step 3 stops at the first rejection, and so does the verify loop of section
 * "Implementation").  The kept drafts and the drawn token are those of the full
 * round; what differs is only what the round can see: a position after the
 * rejection is never checked for non-finite logits, and its p(x_j), q(x_j) are NaN.
 * Draft tokens are still all range-checked.  crop_len[i] = n_i + K_i + 1 is the
 * number of cache entries to keep after the round, n_i = cache_len[i] (0 when
 * cache_len is NULL): the prefix, the last token and the kept drafts (section
 * "Verification attention and the cache"); -1 for an invalid row. */
int oracle_verify_ex(const void *target, const void *draft, int dtype, int64_t V, int32_t B,
                     int64_t n_target_rows, const int32_t *draft_tokens, const float *uniforms,
                     const float *temperature, const int32_t *gamma_per_row, int mode,
                     int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                     double *resid_mass, int32_t *row_status, int32_t *flag_pos, double flag_eps,
                     int nthreads, int early_exit, const int32_t *cache_len, int32_t *crop_len,
                     const int32_t *top_k, const float *top_p, int32_t *flags, int32_t *draw_lo,
                     int32_t *draw_hi)
{
    const double eps = flag_eps > 0 ? flag_eps : 1e-5;
    if (!target || !gamma_per_row || !uniforms || !temperature || !n_accepted || !emitted ||
        V <= 0 || B < 0 || n_target_rows < 0)
        return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32 && dtype != ORACLE_F64)
        return -1;

    /* offsets: exclusive prefix sums of gamma+1 (target rows) and gamma (draft rows) */
    int64_t *t_off = malloc(sizeof(int64_t) * ((size_t)B + 1));
    int64_t *d_off = malloc(sizeof(int64_t) * ((size_t)B + 1));
    if (!t_off || !d_off) {
        free(t_off);
        free(d_off);
        return -1;
    }
    int bad_gamma = 0;
    t_off[0] = d_off[0] = 0;
    for (int32_t i = 0; i < B; ++i) {
        int g = gamma_per_row[i];
        if (g < 0) {
            bad_gamma = 1;
            g = 0;
        }
        t_off[i + 1] = t_off[i] + g + 1;
        d_off[i + 1] = d_off[i] + g;
    }
    if (t_off[B] != n_target_rows)
        bad_gamma = 1;
    if (bad_gamma) {
        for (int32_t i = 0; i < B; ++i) {
            n_accepted[i] = -1;
            if (row_status)
                row_status[i] = ORACLE_BAD_GAMMA;
            if (flag_pos)
                flag_pos[i] = -1;
            if (resid_mass)
                resid_mass[i] = NAN;
            if (crop_len)
                crop_len[i] = -1;
            if (draw_lo)
                draw_lo[i] = -1;
            if (draw_hi)
                draw_hi[i] = -1;
        }
        for (int64_t k = 0; k < n_target_rows; ++k) {
            emitted[k] = -1;
            if (flags)
                flags[k] = 0;
        }
        free(t_off);
        free(d_off);
        return 0;
    }
    if (t_off[B] > B && (!draft || !draft_tokens)) {
        free(t_off);
        free(d_off);
        return -1;
    }

    int rc = 0;
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nth)
    {
        double *P = malloc(sizeof(double) * (size_t)V);
        double *Q = malloc(sizeof(double) * (size_t)V);
        double *w = malloc(sizeof(double) * (size_t)V);
        if (!P || !Q || !w) {
#pragma omp atomic write
            rc = -1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int32_t i = 0; i < B; ++i) {
            if (!P || !Q || !w)
                continue;
            const int g = gamma_per_row[i];
            const int64_t t0 = t_off[i], d0 = d_off[i];
            const double T = (double)temperature[i];
            int status = 0, flag = -1;
            int greedy = mode == ORACLE_GREEDY;
            if (flags)
                for (int j = 0; j <= g; ++j)
                    flags[t0 + j] = 0;
            if (draw_lo)
                draw_lo[i] = -1;
            if (draw_hi)
                draw_hi[i] = -1;
            if (!greedy) {
                if (!isfinite(T))
                    status |= ORACLE_BAD_TEMP;
                else if (T <= 0)
                    greedy = 1;
                else if (T < (double)FLT_MIN)
                    status |= ORACLE_BAD_TEMP;
            }
            for (int j = 0; j < g; ++j) {
                int32_t x = draft_tokens[d0 + j];
                if (x < 0 || (int64_t)x >= V)
                    status |= ORACLE_BAD_TOKEN;
            }
            /* the filters' thresholds at every position (sampling rows with top-k or top-p);
               a top-p boundary within 1e-10 of top_p flags that position */
            double *th_t = NULL, *th_d = NULL;
            const int64_t row_k = top_k ? top_k[i] : 0;
            const double row_p = top_p ? (double)top_p[i] : 1.0;
            if (!greedy && !(status & ORACLE_INVALID_MASK) &&
                ((row_k > 0 && row_k < V) || (row_p > 0 && row_p < 1))) {
                th_t = malloc(sizeof(double) * ((size_t)g + 1));
                th_d = malloc(sizeof(double) * ((size_t)g + 1));
                if (!th_t || !th_d) {
#pragma omp atomic write
                    rc = -1;
                    free(th_t);
                    free(th_d);
                    continue;
                }
                for (int j = 0; j <= g; ++j) {
                    int nt = 0, nd = 0;
                    oracle_filter_threshold(vector_ptr(target, dtype, t0 + j, V), dtype, V, T, row_k, row_p,
                                            1e-10, &th_t[j], &nt);
                    th_d[j] = -INFINITY;
                    if (j < g)
                        oracle_filter_threshold(vector_ptr(draft, dtype, d0 + j, V), dtype, V, T, row_k,
                                                row_p, 1e-10, &th_d[j], &nd);
                    if (nt || nd) {
                        if (flag < 0)
                            flag = j;
                        if (flags)
                            flags[t0 + j] |= ORACLE_FLAG_FILTER;
                    }
                }
            }
#define THETA_T(j) (th_t ? th_t[j] : -INFINITY)
#define THETA_D(j) (th_d ? th_d[j] : -INFINITY)
            /* validity of every position the row reads: all of them, or (early exit) those
               up to the first rejection */
            int K_read = g;
            if (early_exit && !(status & ORACLE_INVALID_MASK)) {
                for (int j = 0; j < g; ++j) {
                    const void *zt = vector_ptr(target, dtype, t0 + j, V);
                    int reject;
                    if (greedy) {
                        reject = (int64_t)draft_tokens[d0 + j] != oracle_argmax(zt, dtype, V);
                    } else {
                        const void *zd = vector_ptr(draft, dtype, d0 + j, V);
                        if (vector_nonfinite(zd, dtype, V)) {
                            K_read = j; /* flagged below, at this position */
                            break;
                        }
                        double px, qx;
                        int q_zero;
                        const double ratio = accept_ratio(zt, zd, dtype, V, T, draft_tokens[d0 + j],
                                                          THETA_T(j), THETA_D(j), &px, &qx, &q_zero);
                        reject = !((double)uniforms[t0 + j] < ratio);
                    }
                    if (vector_nonfinite(zt, dtype, V) || reject) {
                        K_read = j;
                        break;
                    }
                }
            }
            for (int j = 0; j <= K_read && !(status & ORACLE_NONFINITE); ++j)
                if (vector_nonfinite(vector_ptr(target, dtype, t0 + j, V), dtype, V))
                    status |= ORACLE_NONFINITE;
            if (!greedy)
                for (int j = 0; j < g && j <= K_read && !(status & ORACLE_NONFINITE); ++j)
                    if (vector_nonfinite(vector_ptr(draft, dtype, d0 + j, V), dtype, V))
                        status |= ORACLE_NONFINITE;
            if (crop_len)
                crop_len[i] = -1;
            if (status & ORACLE_INVALID_MASK) {
                invalidate_row(n_accepted, emitted, p_x, q_x, resid_mass, i, t0, d0, g);
                if (row_status)
                    row_status[i] = status;
                if (flag_pos)
                    flag_pos[i] = -1;
                free(th_t);
                free(th_d);
                continue;
            }

            if (greedy) {
                /* keep drafts while they equal the target's argmax */
                int K = g;
                for (int j = 0; j < g; ++j) {
                    int64_t a = oracle_argmax(vector_ptr(target, dtype, t0 + j, V), dtype, V);
                    if ((int64_t)draft_tokens[d0 + j] != a) {
                        K = j;
                        break;
                    }
                }
                int64_t aK = oracle_argmax(vector_ptr(target, dtype, t0 + K, V), dtype, V);
                for (int j = 0; j < K; ++j)
                    emitted[t0 + j] = draft_tokens[d0 + j];
                emitted[t0 + K] = (int32_t)aK;
                for (int j = K + 1; j <= g; ++j)
                    emitted[t0 + j] = -1;
                if (draw_lo)
                    draw_lo[i] = (int32_t)aK;
                if (draw_hi)
                    draw_hi[i] = (int32_t)aK;
                n_accepted[i] = K;
                if (crop_len)
                    crop_len[i] = kept_cache_entries(cache_len, i, K);
                if (p_x)
                    for (int j = 0; j < g; ++j)
                        p_x[d0 + j] = NAN;
                if (q_x)
                    for (int j = 0; j < g; ++j)
                        q_x[d0 + j] = NAN;
                if (resid_mass)
                    resid_mass[i] = NAN;
                if (row_status)
                    row_status[i] = status;
                if (flag_pos)
                    flag_pos[i] = -1;
                continue;
            }

            /* p(x_j) and q(x_j) at every draft position */
            int K = g;
            int decided = 0;
            if (early_exit)
                for (int j = 0; j < g; ++j) {
                    if (p_x)
                        p_x[d0 + j] = NAN;
                    if (q_x)
                        q_x[d0 + j] = NAN;
                }
            for (int j = 0; j < g; ++j) {
                if (early_exit && decided)
                    break;
                double px, qx;
                int q_zero;
                const double ratio = accept_ratio(vector_ptr(target, dtype, t0 + j, V),
                                                  vector_ptr(draft, dtype, d0 + j, V), dtype, V, T,
                                                  draft_tokens[d0 + j], THETA_T(j), THETA_D(j), &px, &qx,
                                                  &q_zero);
                if (p_x)
                    p_x[d0 + j] = px;
                if (q_x)
                    q_x[d0 + j] = qx;
                if (q_zero)
                    status |= ORACLE_Q_ZERO;
                if (!decided) {
                    double u = (double)uniforms[t0 + j];
                    if (fabs(u - ratio) < eps) {
                        if (flag < 0)
                            flag = j;
                        if (flags)
                            flags[t0 + j] |= ORACLE_FLAG_NEAR;
                    }
                    if (!(u < ratio)) {
                        K = j;
                        decided = 1;
                    }
                }
            }

            /* residual at a rejection, or p at the bonus position */
            softmax_kept(vector_ptr(target, dtype, t0 + K, V), dtype, V, T, THETA_T(K), P);
            if (K < g) {
                softmax_kept(vector_ptr(draft, dtype, d0 + K, V), dtype, V, T, THETA_D(K), Q);
                double W = 0.0;
                for (int64_t v = 0; v < V; ++v) {
                    w[v] = fmax(0.0, P[v] - Q[v]);
                    W += w[v];
                }
                if (W == 0.0) {
                    memcpy(w, P, sizeof(double) * (size_t)V);
                    status |= ORACLE_ZERO_RESID;
                }
            } else {
                memcpy(w, P, sizeof(double) * (size_t)V);
            }
            double W;
            int near = 0;
            int64_t lo, hi;
            int64_t tok = oracle_inverse_cdf_range(w, V, (double)uniforms[t0 + g], eps, &W, &near, &lo, &hi);
            if (near) {
                if (flag < 0)
                    flag = g;
                if (flags)
                    flags[t0 + g] |= ORACLE_FLAG_NEAR;
            }
            if (draw_lo)
                draw_lo[i] = (int32_t)lo;
            if (draw_hi)
                draw_hi[i] = (int32_t)hi;
            for (int j = 0; j < K; ++j)
                emitted[t0 + j] = draft_tokens[d0 + j];
            emitted[t0 + K] = (int32_t)tok;
            for (int j = K + 1; j <= g; ++j)
                emitted[t0 + j] = -1;
            n_accepted[i] = K;
            if (crop_len)
                crop_len[i] = kept_cache_entries(cache_len, i, K);
            if (resid_mass)
                resid_mass[i] = W;
            if (row_status)
                row_status[i] = status;
            if (flag_pos)
                flag_pos[i] = flag;
            free(th_t);
            free(th_d);
#undef THETA_T
#undef THETA_D
        }
        free(P);
        free(Q);
        free(w);
    }
    free(t_off);
    free(d_off);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* the drafter's draw: one token per logit vector                              */
/* ------------------------------------------------------------------------- */
/* x ~ q with q = softmax(z / T): the drafting step of a round (rayaq.ca
 * "Speculative decoding", section "One round", step 1; the drafter loop of section
 * "Implementation" applies the temperature softmax, then a categorical draw).  The
 * draw is the same inverse CDF as the verification's draws, with the vector's own
 * uniform u_i.  T <= 0 takes the argmax (the greedy drafter of brunomaga.github.io,
 * section "Draft-model speculative decoding"); a non-finite or subnormal positive T
 * and a vector without a softmax make the entry invalid (token -1).  flags[i] = 1
 * when the draw's threshold lies within eps * W of an interior edge of the drawn
 * token's CDF interval; [lo[i], hi[i]] are then the tokens whose interval comes within
 * eps * W of it (lo = hi = the token otherwise). */
int oracle_sample(const void *logits, int dtype, int64_t V, int64_t n, const float *temperature,
                  const float *uniforms, int32_t *tokens, int32_t *status_out, int32_t *flags,
                  double flag_eps, int nthreads, int32_t *lo, int32_t *hi)
{
    const double eps = flag_eps > 0 ? flag_eps : 1e-5;
    if (!logits || !temperature || !uniforms || !tokens || V <= 0 || n < 0)
        return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32 && dtype != ORACLE_F64)
        return -1;
    int rc = 0;
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nth)
    {
        double *w = malloc(sizeof(double) * (size_t)V);
        if (!w) {
#pragma omp atomic write
            rc = -1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            if (!w)
                continue;
            const void *z = vector_ptr(logits, dtype, i, V);
            const double T = (double)temperature[i];
            int status = 0, near = 0;
            int64_t tok = -1, a = -1, b = -1;
            if (!isfinite(T) || (T > 0 && T < (double)FLT_MIN))
                status |= ORACLE_BAD_TEMP;
            if (vector_nonfinite(z, dtype, V))
                status |= ORACLE_NONFINITE;
            if (!status) {
                if (T <= 0) {
                    tok = a = b = oracle_argmax(z, dtype, V);
                } else {
                    oracle_softmax(z, dtype, V, T, w);
                    tok = oracle_inverse_cdf_range(w, V, (double)uniforms[i], eps, NULL, &near, &a, &b);
                }
            }
            tokens[i] = (int32_t)tok;
            if (lo)
                lo[i] = (int32_t)a;
            if (hi)
                hi[i] = (int32_t)b;
            if (status_out)
                status_out[i] = status;
            if (flags)
                flags[i] = near;
        }
        free(w);
    }
    return rc;
}

/* ------------------------------------------------------------------------- */
/* greedy verification of a candidate tree                                     */
/* ------------------------------------------------------------------------- */
/* One forward pass scores every node of a tree of candidate continuations; node
 * k's prediction is the argmax of the target's logits at k, and a node is kept when
 * its parent is kept and its token equals its parent's prediction.  The root (node
 * 0, parent -1) is the target's own token and is always kept.  The result is the
 * longest kept path from the root (brunomaga.github.io "inference-distillation-
 * speculative-decoding", section "Medusa", the tree-verification description), the
 * first such path in node order when several are equally long, followed by the
 * prediction at its last node, the target's next token.  Nodes are listed parents
 * first (parent < node).
 *
 * Tree i holds nodes [off_i, off_i + count_i), off_i = sum_{j<i} count_j; parents[]
 * are tree-local.  Outputs per tree: n_accepted[i] = path length - 1 (the kept
 * drafts); path[off_i + d] = the tree-local node at depth d of the path, -1 after
 * it; emitted[off_i + d] = the path's tokens after the root, then the prediction at
 * its last node, -1 after it.  A tree whose count is below 1, whose root has a
 * parent, or whose node k >= 1 has a parent outside [0, k) is invalid (BAD_TREE);
 * a token outside [0, V) (BAD_TOKEN) or a node vector without a maximum (NaN, +inf,
 * all -inf: NONFINITE) also invalidates the tree; counts that do not add up to
 * n_nodes invalidate every tree (BAD_GAMMA).  An invalid tree gets n_accepted = -1
 * and -1 in every slot. */
int oracle_tree_greedy(const void *logits, int dtype, int64_t V, int32_t B, int64_t n_nodes,
                       const int32_t *counts, const int32_t *tokens, const int32_t *parents,
                       int32_t *n_accepted, int32_t *path, int32_t *emitted, int32_t *status_out,
                       int nthreads)
{
    if (!logits || !counts || !tokens || !parents || !n_accepted || !path || !emitted || V <= 0 ||
        B < 0 || n_nodes < 0)
        return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32 && dtype != ORACLE_F64)
        return -1;
    int64_t *off = malloc(sizeof(int64_t) * ((size_t)B + 1));
    if (!off)
        return -1;
    off[0] = 0;
    int bad_total = 0;
    for (int32_t i = 0; i < B; ++i) {
        int64_t c = counts[i] > 0 ? counts[i] : 0;
        off[i + 1] = off[i] + c;
    }
    if (off[B] != n_nodes)
        bad_total = 1;
    for (int64_t k = 0; k < n_nodes; ++k) {
        path[k] = -1;
        emitted[k] = -1;
    }
    if (bad_total) {
        for (int32_t i = 0; i < B; ++i) {
            n_accepted[i] = -1;
            if (status_out)
                status_out[i] = ORACLE_BAD_GAMMA;
        }
        free(off);
        return 0;
    }
    int rc = 0;
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nth)
    {
        int64_t cap = 0;
        int64_t *pred = NULL, *len = NULL;
#pragma omp for schedule(dynamic, 1)
        for (int32_t i = 0; i < B; ++i) {
            const int64_t o = off[i];
            const int64_t n = off[i + 1] - o;
            int status = 0;
            if (counts[i] < 1 || parents[o] != -1)
                status |= ORACLE_BAD_TREE;
            for (int64_t k = 1; k < n; ++k)
                if (parents[o + k] < 0 || parents[o + k] >= k)
                    status |= ORACLE_BAD_TREE;
            for (int64_t k = 0; k < n; ++k) {
                if (tokens[o + k] < 0 || (int64_t)tokens[o + k] >= V)
                    status |= ORACLE_BAD_TOKEN;
                if (vector_nonfinite(vector_ptr(logits, dtype, o + k, V), dtype, V))
                    status |= ORACLE_NONFINITE;
            }
            if (status_out)
                status_out[i] = status;
            n_accepted[i] = -1;
            if (status)
                continue;
            if (n > cap) {
                free(pred);
                free(len);
                pred = malloc(sizeof(int64_t) * (size_t)n);
                len = malloc(sizeof(int64_t) * (size_t)n);
                cap = n;
                if (!pred || !len) {
#pragma omp atomic write
                    rc = -1;
                    cap = 0;
                    continue;
                }
            }
            /* predictions, then kept nodes in node order: len[k] = kept path length to
               k (0 = not kept) */
            for (int64_t k = 0; k < n; ++k)
                pred[k] = oracle_argmax(vector_ptr(logits, dtype, o + k, V), dtype, V);
            len[0] = 1;
            int64_t best = 0;
            for (int64_t k = 1; k < n; ++k) {
                const int64_t par = parents[o + k];
                len[k] = (len[par] > 0 && (int64_t)tokens[o + k] == pred[par]) ? len[par] + 1 : 0;
                if (len[k] > len[best])
                    best = k;
            }
            /* the path, root first: walk up from its last node */
            const int64_t L = len[best];
            int64_t k = best;
            for (int64_t d = L - 1; d >= 0; --d) {
                path[o + d] = (int32_t)k;
                k = parents[o + k];
            }
            for (int64_t d = 1; d < L; ++d)
                emitted[o + d - 1] = tokens[o + path[o + d]];
            emitted[o + L - 1] = (int32_t)pred[best];
            n_accepted[i] = (int32_t)(L - 1);
        }
        free(pred);
        free(len);
    }
    free(off);
    return rc;
}

int oracle_verify(const void *target, const void *draft, int dtype, int64_t V, int32_t B,
                  int64_t n_target_rows, const int32_t *draft_tokens, const float *uniforms,
                  const float *temperature, const int32_t *gamma_per_row, int mode,
                  int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                  double *resid_mass, int32_t *row_status, int32_t *flag_pos, double flag_eps,
                  int nthreads)
{
    return oracle_verify_ex(target, draft, dtype, V, B, n_target_rows, draft_tokens, uniforms,
                            temperature, gamma_per_row, mode, n_accepted, emitted, p_x, q_x,
                            resid_mass, row_status, flag_pos, flag_eps, nthreads, 0, NULL, NULL, NULL,
                            NULL, NULL, NULL, NULL);
}
