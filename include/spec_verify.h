/*
 * spec_verify: the verification step of speculative sampling on AMD Instinct MI355X
 * (gfx950), as a C ABI.
 *
 * One call verifies a batch of drafted rows.  Row i carries gamma_i drafted tokens
 * x_0 .. x_{gamma_i - 1}, the target model's logits at the gamma_i + 1 positions the
 * verification pass scored, and the drafter's logits at the gamma_i drafted positions.
 * With p_j = softmax(target_j / T_i) and q_j = softmax(draft_j / T_i) (the same
 * temperature for both; brunomaga.github.io "inference-distillation-speculative-
 * decoding", section "Knowledge distillation", the softened-output equation, and
 * rayaq.ca "Speculative decoding", section "Why the output is exactly the target's"):
 *
 *   1. drafts are kept left to right while u_j < min(1, p_j(x_j) / q_j(x_j)); the first
 *      failing j is K (rayaq.ca "Speculative decoding", section "One round", step 3);
 *   2. if K < gamma_i, one token is drawn from the residual
 *      max(0, p_K - q_K) / sum max(0, p_K - q_K) (same section, step 4);
 *   3. if K = gamma_i, one bonus token is drawn from p_{gamma_i} (same section, step 5);
 *   4. in greedy mode drafts are kept while they equal the target's argmax, and the
 *      target's argmax at K is emitted (rayaq.ca "Speculative decoding", section
 *      "The greedy case").
 *
 * A categorical draw with weights w is the inverse CDF in token order: t = u * sum(w),
 * the token is the smallest v whose running sum of w exceeds t.  All randomness is
 * supplied by the caller as uniforms, so the result is a deterministic function of
 * the inputs.
 *
 * LAYOUT (packed rows).  Let t_off[i] = sum_{k<i} (gamma_k + 1) and
 * d_off[i] = sum_{k<i} gamma_k, n_target_rows = sum (gamma_i + 1), n_draft_rows =
 * n_target_rows - batch.  Logit matrices are row-major: target [n_target_rows, vocab],
 * draft [n_draft_rows, vocab]; row t_off[i] + j of target holds position j of batch
 * row i, row d_off[i] + j of draft holds draft position j.  A dense [B, gamma+1, V]
 * target tensor and [B, gamma, V] draft tensor are this layout with a constant gamma.
 *
 * OWNERSHIP.  Every buffer is owned by the caller.  All array pointers are DEVICE
 * pointers (hipMalloc'd or equivalent) unless stated otherwise.  The library keeps no
 * pointer past the call and allocates no device memory: scratch space is the caller's
 * `workspace`, of at least spec_verify_workspace_bytes(...) bytes, 256-byte aligned
 * (spec_verify_noalloc takes it from a fixed device array of the library instead).
 *
 * ASYNCHRONY.  spec_verify enqueues its kernels on `hip_stream` (a hipStream_t; NULL =
 * the null stream) and returns without synchronizing.  Outputs are valid once the
 * stream reaches that point.  Two calls that share a workspace must be ordered on
 * one stream.
 *
 * ERRORS.  Argument errors detectable on the host (null pointers, bad sizes, bad
 * dtype or mode, a workspace that is too small or misaligned, a dense row count that
 * does not match) return a negative sv_status and enqueue nothing.  Data-dependent
 * problems never abort: they are reported per row through row status bits, and an
 * invalid row gets n_accepted = -1 and -1 in all its emitted slots.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_EINVAL = -1,     /* bad pointer, size, mode or layout                     */
    SV_EDTYPE = -2,     /* dtype is not SV_BF16 or SV_F32                         */
    SV_EWORKSPACE = -3, /* workspace too small or not 256-byte aligned            */
    SV_EHIP = -4,       /* the HIP runtime reported an error while enqueueing      */
    SV_ESCRATCH = -5    /* spec_verify_noalloc: the shape needs more workspace than
                           its fixed scratch array holds                           */
} sv_status;

typedef enum { SV_BF16 = 0, SV_F32 = 1 } sv_dtype;
typedef enum { SV_SAMPLE = 0, SV_GREEDY = 1 } sv_mode;

/* Per-row status bits (row_status).  BAD_TOKEN, NONFINITE, BAD_GAMMA, BAD_TEMP and
 * BAD_TREE make a row invalid, and an invalid row carries only those; Q_ZERO and
 * ZERO_RESID describe the decisions of a valid row. */
#define SV_ROW_BAD_TOKEN 1    /* a draft token is outside [0, vocab)                          */
#define SV_ROW_Q_ZERO 2       /* q(x_j) == 0 at some draft position; that ratio is 1 if
                                 p(x_j) > 0, else 0 (informational)                            */
#define SV_ROW_NONFINITE 4    /* a NaN or +inf logit, or a position whose logits are all -inf */
#define SV_ROW_BAD_GAMMA 8    /* some gamma_i < 0, or sum(gamma_i + 1) != n_target_rows; set
                                 on every row of the call                                      */
#define SV_ROW_ZERO_RESID 16  /* zero residual mass at a rejection (only through rounding);
                                 the token was drawn from p_K instead (informational)          */
#define SV_ROW_BAD_TEMP 32    /* sampling row whose temperature is NaN, infinite, or in
                                 (0, FLT_MIN)                                                   */
#define SV_ROW_BAD_TREE 64    /* spec_tree_verify_greedy: a tree with no node, more than 2048
                                 nodes, a root with a parent, or a node whose parent is not an
                                 earlier node of its tree                                      */

/* Optional diagnostics: every pointer may be NULL; all are device pointers. */
typedef struct sv_diag {
    double *p_x;         /* [n_draft_rows]: p_j(x_j) at every draft position of a valid
                            sampling row (NaN elsewhere)                                  */
    double *q_x;         /* [n_draft_rows]: q_j(x_j), likewise                            */
    double *resid_mass;  /* [batch]: sum of the draw weights (residual mass at a
                            rejection, ~1 for a bonus draw); NaN for greedy/invalid rows   */
    int32_t *row_status; /* [batch]: SV_ROW_* bits                                        */
} sv_diag;

/*
 * Bytes of device workspace spec_verify needs for this shape.  Returns 0 for invalid
 * sizes (batch < 0, vocab <= 0, n_target_rows < batch, or dtype not SV_BF16/SV_F32).
 */
size_t spec_verify_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                   int32_t dtype);

/*
 * Verify one batch (see the file comment for what is computed and the layout).
 *
 *   target_logits  [n_target_rows, vocab] dtype   device
 *   draft_logits   [n_draft_rows, vocab]  dtype   device (may be NULL if n_draft_rows == 0)
 *   dtype          SV_BF16 (bf16 bit patterns) or SV_F32
 *   vocab          V, 1 <= V < 2^31
 *   batch          B >= 0 rows
 *   n_target_rows  sum(gamma_i + 1)
 *   draft_tokens   [n_draft_rows] int32 device: x_j of row i at d_off[i] + j
 *   uniforms       [n_target_rows] float device, each in [0, 1): slot t_off[i] + j (j < gamma_i)
 *                  drives accept test j, slot t_off[i] + gamma_i drives the single draw
 *   temperature    [batch] float device: T_i; T_i <= 0 makes row i greedy in SV_SAMPLE mode
 *   gamma_per_row  [batch] int32 device, or NULL for a dense batch where every row has
 *                  `gamma_uniform` drafts (then n_target_rows must be batch*(gamma_uniform+1))
 *   gamma_uniform  used only when gamma_per_row is NULL; >= 0
 *   mode           SV_SAMPLE or SV_GREEDY (greedy ignores temperature and draft_logits)
 *   n_accepted     [batch] int32 device out: K_i, or -1 for an invalid row
 *   emitted_tokens [n_target_rows] int32 device out: row i at t_off[i]: the K_i kept
 *                  drafts, then the drawn (or argmax) token, then -1 up to gamma_i
 *   diag           optional diagnostics (NULL, or a HOST pointer to a struct of device
 *                  pointers)
 *   workspace      device scratch, >= spec_verify_workspace_bytes(...) bytes, 256-aligned;
 *                  its contents need no initialization and are overwritten
 *   hip_stream     hipStream_t to enqueue on
 */
sv_status spec_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
                      int64_t vocab, int32_t batch, int64_t n_target_rows,
                      const int32_t *draft_tokens, const float *uniforms,
                      const float *temperature, const int32_t *gamma_per_row,
                      int32_t gamma_uniform, int32_t mode, int32_t *n_accepted,
                      int32_t *emitted_tokens, const sv_diag *diag, void *workspace,
                      size_t workspace_bytes, void *hip_stream);

/*
 * The drafter's draw: one token per logit vector, x_i ~ q_i = softmax(logits_i / T_i)
 * (rayaq.ca "Speculative decoding", section "One round", step 1, and the drafter loop
 * of section "Implementation", which applies the temperature softmax and then a
 * categorical draw).  The draw is the same inverse CDF as the verification's: with
 * t = u_i * sum_v q_i(v), the token is the smallest v whose running sum of q_i
 * exceeds t.  T_i <= 0 takes the first argmax of the raw logits instead (a greedy
 * drafter, brunomaga.github.io "inference-distillation-speculative-decoding",
 * section "Draft-model speculative decoding").  The logits are read once.
 *
 *   logits       [n, vocab] dtype device, row-major (row i = vector i)
 *   dtype        SV_BF16 or SV_F32
 *   vocab        V, 1 <= V < 2^31
 *   n            vectors, 0 <= n < 2^31
 *   temperature  [n] float device: T_i
 *   uniforms     [n] float device, each in [0, 1): u_i
 *   tokens       [n] int32 device out: the drawn token, or -1 for an invalid vector
 *   row_status   [n] int32 device out, or NULL: SV_ROW_NONFINITE (a NaN or +inf logit,
 *                or all logits -inf) or SV_ROW_BAD_TEMP (T_i NaN, infinite or in
 *                (0, FLT_MIN)); both make the vector invalid
 *   workspace    device scratch, >= spec_sample_workspace_bytes(n, vocab, dtype) bytes,
 *                256-byte aligned, contents overwritten
 *   hip_stream   hipStream_t to enqueue on; asynchronous like spec_verify
 *
 * Host-detectable argument errors return a negative sv_status and enqueue nothing;
 * the caller owns every buffer.
 */
size_t spec_sample_workspace_bytes(int64_t n, int64_t vocab, int32_t dtype);
sv_status spec_sample(const void *logits, int32_t dtype, int64_t vocab, int64_t n,
                      const float *temperature, const float *uniforms, int32_t *tokens,
                      int32_t *row_status, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/*
 * Greedy verification of candidate trees (brunomaga.github.io "inference-distillation-
 * speculative-decoding", section "Medusa": the candidates of several positions form
 * a tree, one forward pass with tree attention scores every node, and the longest
 * accepted path is kept).  Node k's prediction is the first argmax of the target's
 * raw logits at k; a node is kept when its parent is kept and its token equals the
 * parent's prediction; the root (node 0 of a tree, parent -1) is the target's own
 * last token and is always kept.  The result per tree is the longest kept path from
 * the root (the one ending at the lowest node index among equally long ones),
 * followed by the prediction at its last node, the target's next token.
 *
 * LAYOUT.  Trees are packed: tree i holds nodes [off_i, off_i + node_counts[i]),
 * off_i = sum_{j<i} node_counts[j]; row off_i + k of target_logits holds node k of
 * tree i.  parents[] are tree-local node indices, each parent listed before its
 * children (parent < node); the root's parent is -1.
 *
 *   target_logits  [n_nodes, vocab] dtype device
 *   dtype          SV_BF16 or SV_F32
 *   vocab          V, 1 <= V < 2^31
 *   n_trees        B >= 0
 *   n_nodes        sum(node_counts), < 2^31
 *   node_counts    [B] int32 device, each in [1, 2048]
 *   tokens         [n_nodes] int32 device: each node's token (the root's is not tested)
 *   parents        [n_nodes] int32 device
 *   n_accepted     [B] int32 device out: kept drafts on the path (path length - 1), or -1
 *                  for an invalid tree
 *   path           [n_nodes] int32 device out: at off_i + d the tree-local node at depth d
 *                  of the path, then -1
 *   emitted        [n_nodes] int32 device out: at off_i the tokens of the path's nodes
 *                  after the root, then the prediction at its last node, then -1
 *   row_status     [B] int32 device out, or NULL: SV_ROW_BAD_TREE, SV_ROW_BAD_TOKEN (a
 *                  token outside [0, vocab)), SV_ROW_NONFINITE (a node whose logits hold
 *                  NaN or +inf, or are all -inf), SV_ROW_BAD_GAMMA on every tree when the
 *                  counts do not add up to n_nodes; each makes the tree invalid (-1 in all
 *                  its outputs)
 *   workspace      device scratch of spec_tree_verify_greedy_workspace_bytes(...) bytes,
 *                  256-byte aligned, contents overwritten
 *   hip_stream     hipStream_t to enqueue on; asynchronous like spec_verify
 *
 * Every logit is read once.  Host-detectable argument errors return a negative
 * sv_status and enqueue nothing; the caller owns every buffer.
 */
size_t spec_tree_verify_greedy_workspace_bytes(int64_t n_nodes, int64_t vocab, int32_t dtype);
sv_status spec_tree_verify_greedy(const void *target_logits, int32_t dtype, int64_t vocab,
                                  int32_t n_trees, int64_t n_nodes, const int32_t *node_counts,
                                  const int32_t *tokens, const int32_t *parents,
                                  int32_t *n_accepted, int32_t *path, int32_t *emitted,
                                  int32_t *row_status, void *workspace, size_t workspace_bytes,
                                  void *hip_stream);

/*
 * The verification round with early exit: for each row, nothing after its first
 * rejection counts (rayaq.ca "Speculative decoding", section "One round", step 3,
 * which stops at the first rejection).  Kept drafts, drawn tokens and the residual
 * mass are those of spec_verify on the same inputs; what differs is what a row can
 * see: positions after its rejection are not checked for non-finite logits (a NaN
 * there leaves the row valid) and their p(x_j), q(x_j) diagnostics are NaN; a bad
 * draft token anywhere in a row still makes it invalid.  Two plans give identical
 * outputs:
 *   SV_EE_STEPS     positions are read left to right in chunks that double in length:
 *                   step k reads positions [2^k - 1, 2^(k+1) - 1) of both models for
 *                   the rows still undecided, then decides them in order, so
 *                   ceil(log2(gamma_max + 2)) steps cover every row.  A row that
 *                   rejects at K_i reads the vectors of the chunks up to the one
 *                   holding K_i (fewer than 4(K_i + 1)) instead of 2 gamma_i + 1, at
 *                   the price of a fixed cost per step.
 *   SV_EE_ONE_PASS  spec_verify's single streaming pass over every position, with the
 *                   decisions and status bits above: cheaper when the vectors of one
 *                   position are too few to pay for a step.
 *   SV_EE_AUTO      the plan with the smaller expected time for the shape, given the
 *                   caller's per-position acceptance rate (accept_hint); see
 *                   spec_verify_early_exit_plan.
 *
 * The cache rollback (rayaq.ca "Speculative decoding", section "Verification
 * attention and the cache"): a round that keeps K_i drafts over a cached prefix of
 * n_i entries keeps n_i + K_i + 1 entries (the prefix, the last token, the kept
 * drafts) in both models' caches; crop_len[i] receives that length.
 *
 * Arguments as for spec_verify, plus:
 *   gamma_max   ragged batches (gamma_per_row != NULL): a host-side bound on every
 *               gamma_i, >= 0, which sets the number of steps; a row with
 *               gamma_i > gamma_max is invalid (SV_ROW_BAD_GAMMA, n_accepted and
 *               crop_len -1, every emitted slot -1; the chunked plan reads none of its
 *               logits).  Ignored for dense batches (gamma_uniform is the bound).
 *   cache_len   [batch] int32 device, or NULL for n_i = 0: cache entries before the round
 *   crop_len    [batch] int32 device out, or NULL: n_i + K_i + 1, or -1 for an invalid row
 *   plan        SV_EE_AUTO, SV_EE_STEPS or SV_EE_ONE_PASS (else SV_EINVAL)
 *   accept_hint SV_EE_AUTO only: the expected probability that a draft is kept (the
 *               acceptance rate measured on recent rounds, rayaq.ca "Speculative
 *               decoding", section "Tradeoffs"), clamped to [0, 1]; negative or NaN
 *               for the default, 0.6
 *   workspace   >= spec_verify_early_exit_workspace_bytes(...) bytes, 256-byte aligned
 */
#define SV_EE_AUTO 0
#define SV_EE_STEPS 1
#define SV_EE_ONE_PASS 2
size_t spec_verify_early_exit_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                              int32_t dtype);
sv_status spec_verify_early_exit(const void *target_logits, const void *draft_logits, int32_t dtype,
                                 int64_t vocab, int32_t batch, int64_t n_target_rows,
                                 const int32_t *draft_tokens, const float *uniforms,
                                 const float *temperature, const int32_t *gamma_per_row,
                                 int32_t gamma_uniform, int32_t gamma_max, int32_t mode,
                                 const int32_t *cache_len, int32_t *n_accepted,
                                 int32_t *emitted_tokens, int32_t *crop_len, const sv_diag *diag,
                                 int32_t plan, float accept_hint, void *workspace, size_t workspace_bytes,
                                 void *hip_stream);

/*
 * The plan SV_EE_AUTO takes for a shape (SV_EE_STEPS or SV_EE_ONE_PASS), or a negative
 * status for invalid arguments.  Host only, no GPU work.  It compares expected times
 * from rates measured on MI355X: the streaming pass (~6.7 TB/s after ~13 us of fixed
 * cost with its scan) against the steps (~6 TB/s, ~12.5 us fixed per step), where a
 * row reaches chunk k with probability accept_hint^(2^k - 1) and the mean gamma is
 * n_target_rows / batch - 1.
 */
int32_t spec_verify_early_exit_plan(int32_t batch, int64_t n_target_rows, int64_t vocab, int32_t dtype,
                                    int32_t mode, int32_t gamma_max, float accept_hint);

/*
 * The verification round on filtered distributions: each sampling row's top-k and
 * top-p filter is applied to both p and q at every position before the test (rayaq.ca
 * "Speculative decoding", section "Why the output is exactly the target's", last
 * paragraph: the rule preserves exactly the p it is given, so a filter used for
 * sampling must reach both distributions).  A filter keeps the tokens whose logit is
 * at least a threshold theta, and the kept probabilities are renormalized:
 *   top-k (0 < top_k[i] < vocab): theta_k is the top_k-th largest logit counted with
 *         multiplicity, tokens tied with it are kept;
 *   top-p (0 < top_p[i] < 1), applied after top-k: groups of equal logits are taken in
 *         decreasing order until their probability reaches top_p[i]; theta_p is the
 *         logit of the last group taken;
 *   theta = max(theta_k, theta_p); other values of top_k / top_p do not filter.
 * The thresholds are exact (the probability sums behind top-p are taken in fp64 at
 * the exact temperature scale).  A draft token outside the drafter's kept set has
 * q(x) = 0 (SV_ROW_Q_ZERO); one outside the target's kept set has p(x) = 0 and is
 * rejected.  Greedy rows (temperature <= 0) are not filtered.
 *
 * Arguments as for spec_verify in SV_SAMPLE mode, plus:
 *   top_k       [batch] int32 device, or NULL (no top-k)
 *   top_p       [batch] float device, or NULL (no top-p); one of the two must be given
 *   workspace   >= spec_verify_filtered_workspace_bytes(...) bytes, 256-byte aligned
 */
size_t spec_verify_filtered_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                            int32_t dtype);
sv_status spec_verify_filtered(const void *target_logits, const void *draft_logits, int32_t dtype,
                               int64_t vocab, int32_t batch, int64_t n_target_rows,
                               const int32_t *draft_tokens, const float *uniforms,
                               const float *temperature, const int32_t *gamma_per_row,
                               int32_t gamma_uniform, const int32_t *top_k, const float *top_p,
                               int32_t *n_accepted, int32_t *emitted_tokens, const sv_diag *diag,
                               void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * spec_verify without a workspace argument, for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  It enqueues exactly spec_verify's kernels, with the workspace
 * taken from a file-scope device array of SPEC_VERIFY_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends (one copy
 * per device; its address is looked up with hipGetSymbolAddress on the first call on
 * a device).  It calls no hipMalloc, hipFree or other allocating routine.
 *
 * Arguments, layout, outputs and errors as for spec_verify; the workspace and its
 * size are not passed.  A shape whose spec_verify_workspace_bytes(...) exceeds
 * SPEC_VERIFY_NOALLOC_SCRATCH_BYTES returns SV_ESCRATCH and enqueues nothing.
 *
 * Every call on one GPU shares that GPU's scratch array, whose contents need no
 * initialization and are overwritten by each call.  Calls ordered on one stream are
 * safe; calls that may overlap on one GPU (different streams, or different host
 * threads without ordering) race on the array and give undefined results.
 */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES (16u << 20)
sv_status spec_verify_noalloc(const void *target_logits, const void *draft_logits, int32_t dtype,
                              int64_t vocab, int32_t batch, int64_t n_target_rows,
                              const int32_t *draft_tokens, const float *uniforms,
                              const float *temperature, const int32_t *gamma_per_row,
                              int32_t gamma_uniform, int32_t mode, int32_t *n_accepted,
                              int32_t *emitted_tokens, const sv_diag *diag, void *hip_stream);

/* Static, human-readable name of an sv_status value. */
const char *spec_verify_strerror(int32_t status);

/*
 * Profiling aid: when both are non-NULL hipEvent_t handles, every following
 * spec_verify, spec_sample, spec_verify_filtered or spec_tree_verify_greedy call
 * attaches them to the dispatch of its streaming kernel (the statistics pass over
 * every logit), so that
 * hipEventElapsedTime(start_event, stop_event) gives that kernel's own duration;
 * spec_verify_early_exit records them on its stream around its position steps.
 * Pass NULL, NULL to stop.  Process-wide setting, not thread-safe.
 */
sv_status spec_verify_set_profile_events(void *start_event, void *stop_event);

/* Version string of the library. */
const char *spec_verify_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
