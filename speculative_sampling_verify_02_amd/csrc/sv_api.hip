// Host side of the spec_verify C ABI: argument checks, workspace carving and the
// kernel sequence on the caller's stream.  Declarations and the contract are in
// include/spec_verify.h.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

hipEvent_t g_prof_start = nullptr;
hipEvent_t g_prof_stop = nullptr;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" size_t spec_verify_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                              int32_t dtype)
{
    if (batch < 0 || vocab <= 0 || vocab > INT32_MAX || n_target_rows < batch ||
        (dtype != SV_BF16 && dtype != SV_F32))
        return 0;
    if (2 * n_target_rows - batch > INT32_MAX) return 0;
    return sv::make_layout(batch, n_target_rows, vocab, dtype).total;
}

extern "C" const char *spec_verify_strerror(int32_t status)
{
    switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (pointer, size, mode or layout)";
    case SV_EDTYPE: return "unsupported dtype (expected SV_BF16 or SV_F32)";
    case SV_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case SV_EHIP: return "HIP runtime error while enqueueing kernels";
    case SV_ESCRATCH: return "shape needs more workspace than spec_verify_noalloc's fixed scratch array";
    default: return "unknown status";
    }
}

extern "C" const char *spec_verify_version(void) { return "spec_verify 0.1 (gfx950)"; }

extern "C" sv_status spec_verify_set_profile_events(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr)) return SV_EINVAL;
    g_prof_start = static_cast<hipEvent_t>(start_event);
    g_prof_stop = static_cast<hipEvent_t>(stop_event);
    return SV_OK;
}

// The round with early exit run as one pass (its decisions from a pass that read
// every position): what the scan needs besides spec_verify's arguments.
struct EeArgs {
    const int32_t *cache_len;
    int32_t *crop_len;
    int32_t gamma_max;
};

static sv_status verify_impl(const void *target_logits, const void *draft_logits, int32_t dtype,
                             int64_t vocab, int32_t batch, int64_t n_target_rows,
                             const int32_t *draft_tokens, const float *uniforms,
                             const float *temperature, const int32_t *gamma_per_row,
                             int32_t gamma_uniform, int32_t mode, int32_t *n_accepted,
                             int32_t *emitted_tokens, const sv_diag *diag, void *workspace,
                             size_t workspace_bytes, void *hip_stream, const int32_t *top_k,
                             const float *top_p, const EeArgs *ee = nullptr)
{
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    if (mode != SV_SAMPLE && mode != SV_GREEDY) return SV_EINVAL;
    if (batch < 0 || vocab <= 0 || vocab > INT32_MAX || n_target_rows < batch) return SV_EINVAL;
    if (2 * n_target_rows - batch > INT32_MAX) return SV_EINVAL;
    if (gamma_per_row == nullptr) {
        if (gamma_uniform < 0) return SV_EINVAL;
        if (n_target_rows != (int64_t)batch * ((int64_t)gamma_uniform + 1)) return SV_EINVAL;
    }
    if (batch == 0) return n_target_rows == 0 ? SV_OK : SV_EINVAL;
    const int64_t n_draft_rows = n_target_rows - batch;
    if (!target_logits || !uniforms || !temperature || !n_accepted || !emitted_tokens || !workspace)
        return SV_EINVAL;
    if (n_draft_rows > 0 && (!draft_tokens || (mode == SV_SAMPLE && !draft_logits))) return SV_EINVAL;

    const sv::Layout L = sv::make_layout(batch, n_target_rows, vocab, dtype);
    const bool filtered = top_k != nullptr || top_p != nullptr;
    const size_t theta_bytes = filtered ? sv::align256(sizeof(float) * (size_t)(2 * n_target_rows - batch)) : 0;
    // the maxima of 64-logit units, when the threshold search can take them
    const bool units = filtered && sv::filter_units_num(vocab) != 0;
    const size_t umax_bytes = units ? sv::filter_umax_bytes(batch, n_target_rows, vocab) : 0;
    if (filtered && mode != SV_SAMPLE) return SV_EINVAL;
    if (workspace_bytes < L.total + theta_bytes + umax_bytes || ((uintptr_t)workspace & 255u) != 0)
        return SV_EWORKSPACE;

    // 16-byte vector loads need every logit row to start 16-byte aligned
    const int64_t esz = dtype == SV_BF16 ? 2 : 4;
    const bool aligned = (vocab * esz) % 16 == 0 && aligned16(target_logits) &&
                         (n_draft_rows == 0 || draft_logits == nullptr || aligned16(draft_logits));

    char *ws = static_cast<char *>(workspace);
    sv::Params P{};
    P.target = target_logits;
    P.draft = draft_logits;
    P.V = vocab;
    P.B = batch;
    P.mode = mode;
    P.nT = n_target_rows;
    P.nD = n_draft_rows;
    P.tokens = draft_tokens;
    P.uniforms = uniforms;
    P.temperature = temperature;
    P.gamma = gamma_per_row;
    P.gamma_uniform = gamma_per_row ? 0 : gamma_uniform;
    P.n_accepted = n_accepted;
    P.emitted = emitted_tokens;
    if (diag) {
        P.p_x = diag->p_x;
        P.q_x = diag->q_x;
        P.resid = diag->resid_mass;
        P.row_status = diag->row_status;
    }
    P.hdr = reinterpret_cast<sv::Header *>(ws + L.hdr);
    P.rows = reinterpret_cast<sv::RowInfo *>(ws + L.rows);
    P.vinfo = reinterpret_cast<sv::VecInfo *>(ws + L.vinfo);
    P.parts = reinterpret_cast<sv::Partial *>(ws + L.parts);
    P.zx = reinterpret_cast<float *>(ws + L.zx);
    P.draws = reinterpret_cast<sv::RowDraw *>(ws + L.draws);
    P.tiles = reinterpret_cast<sv::Sum2 *>(ws + L.tiles);
    P.geo = sv::make_geometry(batch, n_target_rows, vocab, mode, dtype, sv::stats_grid_cap(dtype, aligned));
    if (!gamma_per_row) {
        P.geo.inv_t = 1.0 / ((double)gamma_uniform + 1.0);
        P.geo.inv_d = gamma_uniform > 0 ? 1.0 / (double)gamma_uniform : 0.0;
    }
    if (filtered) {
        P.top_k = top_k;
        P.top_p = top_p;
        P.theta = reinterpret_cast<float *>(ws + L.total);
        if (units) P.umax = reinterpret_cast<uint16_t *>(ws + L.total + theta_bytes);
    }
    if (ee) {
        P.cache_len = ee->cache_len;
        P.crop_len = ee->crop_len;
        P.gamma_max = ee->gamma_max;
    }

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipSuccess;
    if (gamma_per_row) e = sv::launch_prepare(P, s);
    // filtered calls: the streaming pass also stores the maximum of every 64 consecutive
    // logits, from which the threshold search bounds the top-k and reads only the units
    // that can hold it
    if (e == hipSuccess) e = sv::launch_stats(P, s, dtype, aligned, g_prof_start, g_prof_stop);
    if (e == hipSuccess && filtered)
        e = units ? sv::launch_filter_units(P, s, dtype, aligned) : sv::launch_filter(P, s, dtype, aligned);
    // bf16 sampling: the accept scan and the residual's tile sums in one kernel; otherwise
    // the scan, then (sampling) the tile sums
    if (e == hipSuccess) {
        if (mode == SV_SAMPLE && dtype == 0) {
            P.st_split = sv::scan_tiles_split(batch, P.geo.ntiles);
            e = sv::launch_scan_tiles(P, s, aligned, ee != nullptr);
        } else {
            e = sv::launch_scan(P, s, dtype, ee != nullptr);
            if (e == hipSuccess && mode == SV_SAMPLE) e = sv::launch_verify(P, s, dtype, aligned);
        }
    }
    if (e == hipSuccess && mode == SV_SAMPLE) e = sv::launch_draw_final(P, s, dtype, aligned);
    return e == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" sv_status spec_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
                                 int64_t vocab, int32_t batch, int64_t n_target_rows,
                                 const int32_t *draft_tokens, const float *uniforms,
                                 const float *temperature, const int32_t *gamma_per_row,
                                 int32_t gamma_uniform, int32_t mode, int32_t *n_accepted,
                                 int32_t *emitted_tokens, const sv_diag *diag, void *workspace,
                                 size_t workspace_bytes, void *hip_stream)
{
    return verify_impl(target_logits, draft_logits, dtype, vocab, batch, n_target_rows, draft_tokens, uniforms,
                       temperature, gamma_per_row, gamma_uniform, mode, n_accepted, emitted_tokens, diag,
                       workspace, workspace_bytes, hip_stream, nullptr, nullptr);
}

extern "C" size_t spec_verify_filtered_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                                       int32_t dtype)
{
    const size_t base = spec_verify_workspace_bytes(batch, n_target_rows, vocab, dtype);
    if (base == 0) return 0;
    const size_t umax = sv::filter_units_num(vocab) ? sv::filter_umax_bytes(batch, n_target_rows, vocab) : 0;
    return base + sv::align256(sizeof(float) * (size_t)(2 * n_target_rows - batch)) + umax;
}

// The round on filtered distributions: the streaming pass also stores the maximum of
// every 64 consecutive logits of the vectors whose rows filter (and skips their sums),
// and the threshold search then gives each such vector its threshold and its record
// over the kept logits (filter_units_kernel; filter_kernel beyond 524288 logits); the
// scan and the draws then see the filtered p and q.
extern "C" sv_status spec_verify_filtered(const void *target_logits, const void *draft_logits, int32_t dtype,
                                          int64_t vocab, int32_t batch, int64_t n_target_rows,
                                          const int32_t *draft_tokens, const float *uniforms,
                                          const float *temperature, const int32_t *gamma_per_row,
                                          int32_t gamma_uniform, const int32_t *top_k, const float *top_p,
                                          int32_t *n_accepted, int32_t *emitted_tokens, const sv_diag *diag,
                                          void *workspace, size_t workspace_bytes, void *hip_stream)
{
    if (top_k == nullptr && top_p == nullptr) return SV_EINVAL;
    return verify_impl(target_logits, draft_logits, dtype, vocab, batch, n_target_rows, draft_tokens, uniforms,
                       temperature, gamma_per_row, gamma_uniform, SV_SAMPLE, n_accepted, emitted_tokens, diag,
                       workspace, workspace_bytes, hip_stream, top_k, top_p);
}

extern "C" size_t spec_sample_workspace_bytes(int64_t n, int64_t vocab, int32_t dtype)
{
    if (n < 0 || n > INT32_MAX || vocab <= 0 || vocab > INT32_MAX || (dtype != SV_BF16 && dtype != SV_F32))
        return 0;
    const sv::Layout L = sv::make_layout((int32_t)n, n, vocab, dtype);
    return L.total + ((sizeof(int32_t) * (size_t)n + 255) & ~(size_t)255);
}

// The drafter's draw is a verification of rows without drafts: every row is one
// position, whose bonus draw from p_0 = softmax(z / T) with the row's uniform is the
// sampled token (or its argmax when T <= 0).  No second pass over the logits runs:
// the draw reuses the streaming pass's piece sums.
extern "C" sv_status spec_sample(const void *logits, int32_t dtype, int64_t vocab, int64_t n,
                                 const float *temperature, const float *uniforms, int32_t *tokens,
                                 int32_t *row_status, void *workspace, size_t workspace_bytes,
                                 void *hip_stream)
{
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    if (n < 0 || n > INT32_MAX || vocab <= 0 || vocab > INT32_MAX) return SV_EINVAL;
    if (n == 0) return SV_OK;
    if (!logits || !temperature || !uniforms || !tokens || !workspace) return SV_EINVAL;
    const size_t need = spec_sample_workspace_bytes(n, vocab, dtype);
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return SV_EWORKSPACE;

    const sv::Layout L = sv::make_layout((int32_t)n, n, vocab, dtype);
    const int64_t esz = dtype == SV_BF16 ? 2 : 4;
    const bool aligned = (vocab * esz) % 16 == 0 && aligned16(logits);
    char *ws = static_cast<char *>(workspace);
    sv::Params P{};
    P.target = logits;
    P.V = vocab;
    P.B = (int32_t)n;
    P.mode = SV_SAMPLE;
    P.nT = n;
    P.nD = 0;
    P.uniforms = uniforms;
    P.temperature = temperature;
    P.gamma_uniform = 0;
    P.n_accepted = reinterpret_cast<int32_t *>(ws + L.total);
    P.emitted = tokens;
    P.row_status = row_status;
    P.hdr = reinterpret_cast<sv::Header *>(ws + L.hdr);
    P.rows = reinterpret_cast<sv::RowInfo *>(ws + L.rows);
    P.vinfo = reinterpret_cast<sv::VecInfo *>(ws + L.vinfo);
    P.parts = reinterpret_cast<sv::Partial *>(ws + L.parts);
    P.zx = reinterpret_cast<float *>(ws + L.zx);
    P.draws = reinterpret_cast<sv::RowDraw *>(ws + L.draws);
    P.tiles = reinterpret_cast<sv::Sum2 *>(ws + L.tiles);
    P.geo = sv::make_geometry((int32_t)n, n, vocab, SV_SAMPLE, dtype, sv::stats_grid_cap(dtype, aligned));
    P.geo.inv_t = 1.0;
    P.geo.inv_d = 0.0;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = sv::launch_stats(P, s, dtype, aligned, g_prof_start, g_prof_stop);
    if (e == hipSuccess) e = sv::launch_scan_draw(P, s, dtype, aligned);
    return e == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" size_t spec_tree_verify_greedy_workspace_bytes(int64_t n_nodes, int64_t vocab, int32_t dtype)
{
    if (n_nodes < 0 || n_nodes > INT32_MAX || vocab <= 0 || vocab > INT32_MAX ||
        (dtype != SV_BF16 && dtype != SV_F32))
        return 0;
    return sv::make_layout((int32_t)n_nodes, n_nodes, vocab, dtype).total;
}

// Greedy tree verification: the streaming pass in greedy mode over every node's
// vector (a call whose rows are the nodes, each without drafts), then one workgroup
// per tree.
extern "C" sv_status spec_tree_verify_greedy(const void *target_logits, int32_t dtype, int64_t vocab,
                                             int32_t n_trees, int64_t n_nodes, const int32_t *node_counts,
                                             const int32_t *tokens, const int32_t *parents,
                                             int32_t *n_accepted, int32_t *path, int32_t *emitted,
                                             int32_t *row_status, void *workspace, size_t workspace_bytes,
                                             void *hip_stream)
{
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    if (n_trees < 0 || n_nodes < 0 || n_nodes > INT32_MAX || vocab <= 0 || vocab > INT32_MAX) return SV_EINVAL;
    if (n_trees == 0) return n_nodes == 0 ? SV_OK : SV_EINVAL;
    if (!target_logits && n_nodes > 0) return SV_EINVAL;
    if (!node_counts || !tokens || !parents || !n_accepted || !path || !emitted || !workspace) return SV_EINVAL;
    const size_t need = spec_tree_verify_greedy_workspace_bytes(n_nodes, vocab, dtype);
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return SV_EWORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int64_t esz = dtype == SV_BF16 ? 2 : 4;
    const bool aligned = (vocab * esz) % 16 == 0 && aligned16(target_logits);
    const sv::Layout L = sv::make_layout((int32_t)n_nodes, n_nodes, vocab, dtype);
    char *ws = static_cast<char *>(workspace);
    hipError_t e = hipSuccess;
    if (n_nodes > 0) {
        sv::Params P{};
        P.target = target_logits;
        P.V = vocab;
        P.B = (int32_t)n_nodes;
        P.mode = SV_GREEDY;
        P.nT = n_nodes;
        P.nD = 0;
        P.gamma_uniform = 0;
        P.hdr = reinterpret_cast<sv::Header *>(ws + L.hdr);
        P.parts = reinterpret_cast<sv::Partial *>(ws + L.parts);
        P.zx = reinterpret_cast<float *>(ws + L.zx);
        P.geo = sv::make_geometry((int32_t)n_nodes, n_nodes, vocab, SV_GREEDY, dtype,
                                  sv::stats_grid_cap(dtype, aligned));
        P.geo.inv_t = 1.0;
        P.geo.inv_d = 0.0;
        e = sv::launch_stats(P, s, dtype, aligned, g_prof_start, g_prof_stop);
    }
    sv::TreeParams T{};
    T.parts = reinterpret_cast<const sv::Partial *>(ws + L.parts);
    T.ipv = sv::ceil_div(vocab, 2 * sv::item_elems(dtype));
    T.V = vocab;
    T.n_nodes = n_nodes;
    T.B = n_trees;
    T.counts = node_counts;
    T.tokens = tokens;
    T.parents = parents;
    T.n_accepted = n_accepted;
    T.path = path;
    T.emitted = emitted;
    T.row_status = row_status;
    if (e == hipSuccess) e = sv::launch_tree(T, s);
    return e == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" size_t spec_verify_early_exit_workspace_bytes(int32_t batch, int64_t n_target_rows, int64_t vocab,
                                                         int32_t dtype)
{
    const size_t base = spec_verify_workspace_bytes(batch, n_target_rows, vocab, dtype);
    return base == 0 ? 0 : base + sv::early_exit_extra_bytes(batch, n_target_rows);
}

// Expected time of the two plans of the round with early exit, from rates measured on
// MI355X: the streaming pass reads at ~6.7 TB/s after ~8 us of start-up, a step of the
// chunked plan reads at ~6 TB/s and pays ~12.5 us for its two launches and their
// dependent loads, and the one-pass plan's scan costs ~5 us more than the steps'
// decisions do.  The residual's tile sums and the draw are the same in both.  With a
// per-position acceptance rate alpha, chunk k (positions [2^k - 1, 2^(k+1) - 1)) is
// reached by a row with probability alpha^(2^k - 1).
static int32_t ee_choose(int32_t batch, int64_t n_target_rows, int64_t vocab, int32_t dtype, int32_t mode,
                         int32_t gamma_max, float accept_hint)
{
    constexpr double kPassRate = 6.7e12, kPassFixed = 8e-6 + 5e-6;
    constexpr double kStepRate = 6.0e12, kStepFixed = 12.5e-6;
    constexpr double kDefaultAlpha = 0.6;
    double alpha = accept_hint >= 0.0f ? (double)accept_hint : kDefaultAlpha;   // NaN: the default
    if (alpha > 1.0) alpha = 1.0;
    const double esz = dtype == SV_BF16 ? 2.0 : 4.0;
    const double vec_bytes = (double)vocab * esz;
    const bool sample = mode == SV_SAMPLE;
    const double n_vecs = (double)n_target_rows + (sample ? (double)(n_target_rows - batch) : 0.0);
    const double t_pass = kPassFixed + n_vecs * vec_bytes / kPassRate;
    const double gbar = (double)n_target_rows / (double)batch - 1.0;   // mean drafts per row
    double t_steps = 0.0;
    for (int k = 0; k < 62; ++k) {
        const double j0 = (double)((int64_t(1) << k) - 1);
        if (j0 > (double)gamma_max) break;
        const double j1 = (double)((int64_t(1) << (k + 1)) - 1);
        const double nt = std::max(0.0, std::min(j1, gbar + 1.0) - j0);
        const double nd = sample ? std::max(0.0, std::min(j1, gbar) - j0) : 0.0;
        t_steps += kStepFixed + (double)batch * std::pow(alpha, j0) * (nt + nd) * vec_bytes / kStepRate;
    }
    return t_steps < t_pass ? SV_EE_STEPS : SV_EE_ONE_PASS;
}

extern "C" int32_t spec_verify_early_exit_plan(int32_t batch, int64_t n_target_rows, int64_t vocab, int32_t dtype,
                                               int32_t mode, int32_t gamma_max, float accept_hint)
{
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    if (mode != SV_SAMPLE && mode != SV_GREEDY) return SV_EINVAL;
    if (batch <= 0 || vocab <= 0 || n_target_rows < batch || gamma_max < 0) return SV_EINVAL;
    return ee_choose(batch, n_target_rows, vocab, dtype, mode, gamma_max, accept_hint);
}

// The round with early exit.  SV_EE_STEPS: step k reads positions
// [2^k - 1, 2^(k+1) - 1) of the rows still undecided (a listed-vector streaming
// kernel), then decides them in order (one workgroup per listed row).  SV_EE_ONE_PASS:
// spec_verify's kernels, the scan with early-exit semantics.  The draws follow as in
// spec_verify.
extern "C" sv_status spec_verify_early_exit(const void *target_logits, const void *draft_logits, int32_t dtype,
                                            int64_t vocab, int32_t batch, int64_t n_target_rows,
                                            const int32_t *draft_tokens, const float *uniforms,
                                            const float *temperature, const int32_t *gamma_per_row,
                                            int32_t gamma_uniform, int32_t gamma_max, int32_t mode,
                                            const int32_t *cache_len, int32_t *n_accepted,
                                            int32_t *emitted_tokens, int32_t *crop_len, const sv_diag *diag,
                                            int32_t plan, float accept_hint, void *workspace,
                                            size_t workspace_bytes, void *hip_stream)
{
    if (plan != SV_EE_AUTO && plan != SV_EE_STEPS && plan != SV_EE_ONE_PASS) return SV_EINVAL;
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    if (mode != SV_SAMPLE && mode != SV_GREEDY) return SV_EINVAL;
    if (batch < 0 || vocab <= 0 || vocab > INT32_MAX || n_target_rows < batch) return SV_EINVAL;
    if (2 * n_target_rows - batch > INT32_MAX) return SV_EINVAL;
    if (gamma_per_row == nullptr) {
        if (gamma_uniform < 0) return SV_EINVAL;
        if (n_target_rows != (int64_t)batch * ((int64_t)gamma_uniform + 1)) return SV_EINVAL;
        gamma_max = gamma_uniform;
    } else if (gamma_max < 0) {
        return SV_EINVAL;
    }
    if (batch == 0) return n_target_rows == 0 ? SV_OK : SV_EINVAL;
    const int64_t n_draft_rows = n_target_rows - batch;
    if (!target_logits || !uniforms || !temperature || !n_accepted || !emitted_tokens || !workspace)
        return SV_EINVAL;
    if (n_draft_rows > 0 && (!draft_tokens || (mode == SV_SAMPLE && !draft_logits))) return SV_EINVAL;
    const size_t need = spec_verify_early_exit_workspace_bytes(batch, n_target_rows, vocab, dtype);
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return SV_EWORKSPACE;
    if (plan == SV_EE_AUTO) plan = ee_choose(batch, n_target_rows, vocab, dtype, mode, gamma_max, accept_hint);
    if (plan == SV_EE_ONE_PASS) {
        const EeArgs ee{cache_len, crop_len, gamma_max};
        return verify_impl(target_logits, draft_logits, dtype, vocab, batch, n_target_rows, draft_tokens, uniforms,
                           temperature, gamma_per_row, gamma_uniform, mode, n_accepted, emitted_tokens, diag,
                           workspace, workspace_bytes, hip_stream, nullptr, nullptr, &ee);
    }

    const int64_t esz = dtype == SV_BF16 ? 2 : 4;
    const bool aligned = (vocab * esz) % 16 == 0 && aligned16(target_logits) &&
                         (n_draft_rows == 0 || draft_logits == nullptr || aligned16(draft_logits));
    const sv::Layout L = sv::make_layout(batch, n_target_rows, vocab, dtype);
    char *ws = static_cast<char *>(workspace);
    sv::Params P{};
    P.target = target_logits;
    P.draft = draft_logits;
    P.V = vocab;
    P.B = batch;
    P.mode = mode;
    P.nT = n_target_rows;
    P.nD = n_draft_rows;
    P.tokens = draft_tokens;
    P.uniforms = uniforms;
    P.temperature = temperature;
    P.gamma = gamma_per_row;
    P.gamma_uniform = gamma_per_row ? 0 : gamma_uniform;
    P.n_accepted = n_accepted;
    P.emitted = emitted_tokens;
    if (diag) {
        P.p_x = diag->p_x;
        P.q_x = diag->q_x;
        P.resid = diag->resid_mass;
        P.row_status = diag->row_status;
    }
    P.hdr = reinterpret_cast<sv::Header *>(ws + L.hdr);
    P.rows = reinterpret_cast<sv::RowInfo *>(ws + L.rows);
    P.vinfo = reinterpret_cast<sv::VecInfo *>(ws + L.vinfo);
    P.parts = reinterpret_cast<sv::Partial *>(ws + L.parts);
    P.zx = reinterpret_cast<float *>(ws + L.zx);
    P.draws = reinterpret_cast<sv::RowDraw *>(ws + L.draws);
    P.tiles = reinterpret_cast<sv::Sum2 *>(ws + L.tiles);
    P.geo = sv::make_geometry(batch, n_target_rows, vocab, mode, dtype, sv::stats_grid_cap(dtype, aligned));
    if (!gamma_per_row) {
        P.geo.inv_t = 1.0 / ((double)gamma_uniform + 1.0);
        P.geo.inv_d = gamma_uniform > 0 ? 1.0 / (double)gamma_uniform : 0.0;
    }
    char *ex = ws + L.total;
    const size_t cap = sv::early_exit_list_cap(batch, n_target_rows);
    const size_t rows_b = sv::align256(sizeof(int32_t) * 2 * (size_t)batch);
    const size_t vecs_b = sv::align256(sizeof(int32_t) * 2 * cap);
    const size_t cnt_b = sv::align256(sizeof(int32_t) * 4);
    P.ee_rows[0] = reinterpret_cast<int32_t *>(ex);
    P.ee_rows[1] = P.ee_rows[0] + batch;
    P.ee_vecs[0] = reinterpret_cast<int32_t *>(ex + rows_b);
    P.ee_vecs[1] = P.ee_vecs[0] + cap;
    P.ee_count = reinterpret_cast<int32_t *>(ex + rows_b + vecs_b);
    P.ee_status = reinterpret_cast<int32_t *>(ex + rows_b + vecs_b + cnt_b);
    P.cache_len = cache_len;
    P.crop_len = crop_len;
    P.gamma_max = gamma_max;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipSuccess;
    if (gamma_per_row) e = sv::launch_prepare(P, s);
    if (e == hipSuccess) e = sv::launch_ee_init(P, s);
    if (e == hipSuccess && g_prof_start) e = hipEventRecord(g_prof_start, s);
    // chunks of positions [2^k - 1, 2^(k+1) - 1) up to gamma_max
    const int64_t vec_per_pos = mode == SV_SAMPLE ? 2 : 1;
    const int64_t n_vecs = mode == SV_SAMPLE ? 2 * n_target_rows - batch : n_target_rows;
    for (int k = 0; e == hipSuccess; ++k) {
        const int64_t j0 = (int64_t(1) << k) - 1;
        if (j0 > gamma_max) break;
        const int64_t j1 = std::min<int64_t>((int64_t(1) << (k + 1)) - 1, (int64_t)gamma_max + 1);
        const int64_t j2 = std::min<int64_t>((int64_t(1) << (k + 2)) - 1, (int64_t)gamma_max + 1);
        P.step = k;
        P.ee_j0 = (int32_t)j0;
        P.ee_j1 = (int32_t)j1;
        P.ee_j2 = (int32_t)j2;
        const int64_t max_vecs = k == 0 ? vec_per_pos * batch : std::min(n_vecs, vec_per_pos * batch * (j1 - j0));
        e = sv::launch_stats_list(P, s, dtype, aligned, max_vecs);
        if (e == hipSuccess) e = sv::launch_ee_step(P, s, dtype);
    }
    if (e == hipSuccess && g_prof_stop) e = hipEventRecord(g_prof_stop, s);
    if (e == hipSuccess && mode == SV_SAMPLE) e = sv::launch_verify(P, s, dtype, aligned);
    if (e == hipSuccess && mode == SV_SAMPLE) e = sv::launch_draw_final(P, s, dtype, aligned);
    return e == hipSuccess ? SV_OK : SV_EHIP;
}
