/*
 * fp64 CPU oracle of the speculative-sampling verification step: declarations.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline); see oracle.c.
 * This header is the oracle's own and is not shared with the HIP path.
 */
#ifndef SPEC_VERIFY_ORACLE_H
#define SPEC_VERIFY_ORACLE_H
#include <stdint.h>

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };
enum { ORACLE_SAMPLE = 0, ORACLE_GREEDY = 1 };

/* per-row status bits */
#define ORACLE_BAD_TOKEN 1   /* a draft token outside [0, V)                        */
#define ORACLE_Q_ZERO 2      /* q(x) == 0 at some draft position (informational)   */
#define ORACLE_NONFINITE 4   /* NaN / +inf logit, or a position with all -inf       */
#define ORACLE_BAD_GAMMA 8   /* gamma < 0, or sum(gamma+1) != n_target_rows        */
#define ORACLE_ZERO_RESID 16 /* zero residual mass at a rejection (informational)  */
#define ORACLE_BAD_TEMP 32   /* sampling row with non-finite or subnormal T         */
#define ORACLE_BAD_TREE 64   /* a tree whose parents are not listed before children */
/* per-decision flags (oracle_verify_ex flags[]) */
#define ORACLE_FLAG_NEAR 1   /* the decision lies within eps of its threshold            */
#define ORACLE_FLAG_FILTER 2 /* a top-p boundary within 1e-10 at this position           */
#define ORACLE_INVALID_MASK (ORACLE_BAD_TOKEN | ORACLE_NONFINITE | ORACLE_BAD_GAMMA | ORACLE_BAD_TEMP | ORACLE_BAD_TREE)

int oracle_softmax(const void *z, int dtype, int64_t V, double T, double *p);
int64_t oracle_argmax(const void *z, int dtype, int64_t V);
int oracle_position(const void *zt, const void *zd, int dtype, int64_t V, double T, double *p,
                    double *q, double *alpha, double *resid_mass, double *residual);
int64_t oracle_inverse_cdf(const double *w, int64_t V, double u, double eps, double *W_out,
                           int *near_edge);
int64_t oracle_inverse_cdf_range(const double *w, int64_t V, double u, double eps, double *W_out,
                                 int *near_edge, int64_t *lo, int64_t *hi);
int oracle_verify(const void *target, const void *draft, int dtype, int64_t V, int32_t B,
                  int64_t n_target_rows, const int32_t *draft_tokens, const float *uniforms,
                  const float *temperature, const int32_t *gamma_per_row, int mode,
                  int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                  double *resid_mass, int32_t *row_status, int32_t *flag_pos, double flag_eps,
                  int nthreads);
int oracle_sample(const void *logits, int dtype, int64_t V, int64_t n, const float *temperature,
                  const float *uniforms, int32_t *tokens, int32_t *status_out, int32_t *flags,
                  double flag_eps, int nthreads, int32_t *lo, int32_t *hi);
int oracle_tree_greedy(const void *logits, int dtype, int64_t V, int32_t B, int64_t n_nodes,
                       const int32_t *counts, const int32_t *tokens, const int32_t *parents,
                       int32_t *n_accepted, int32_t *path, int32_t *emitted, int32_t *status_out,
                       int nthreads);
int oracle_verify_ex(const void *target, const void *draft, int dtype, int64_t V, int32_t B,
                     int64_t n_target_rows, const int32_t *draft_tokens, const float *uniforms,
                     const float *temperature, const int32_t *gamma_per_row, int mode,
                     int32_t *n_accepted, int32_t *emitted, double *p_x, double *q_x,
                     double *resid_mass, int32_t *row_status, int32_t *flag_pos, double flag_eps,
                     int nthreads, int early_exit, const int32_t *cache_len, int32_t *crop_len,
                     const int32_t *top_k, const float *top_p, int32_t *flags, int32_t *draw_lo,
                     int32_t *draw_hi);
int oracle_filter_threshold(const void *z, int dtype, int64_t V, double T, int64_t top_k, double top_p,
                            double eps, double *theta_out, int *near);
#endif
