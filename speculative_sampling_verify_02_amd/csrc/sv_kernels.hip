// The kernels after the streaming pass of the speculative-sampling verification step.
//
// prepare_kernel turns a ragged batch's draft counts into packed offsets and the
// per-vector table the streaming pass reads.  scan_kernel (one workgroup per row)
// merges a row's piece records per vector and runs the accept scan over the
// positions: it keeps x_j while u_j < min(1, p_j(x_j)/q_j(x_j)) (rayaq.ca
// "Speculative decoding", section "One round", step 3), or while x_j equals the
// argmax in greedy mode (section "The greedy case"), writes the row's outputs and
// what its draw needs.  After a rejection verify_kernel re-reads position K of the
// row and sums the residual max(0, p - q) (step 4) per 512-logit tile, and
// draw_final_kernel walks the tile sums and one tile to the inverse-CDF token.  For
// bf16 sampling scan_tiles_kernel does the scan and the tile sums in one launch:
// several workgroups per row each run the row's scan (the same arithmetic, so the
// same K) and then sum their share of the row's tiles.  The bonus token (step 5) is
// drawn from p, whose sums per piece the streaming pass already holds:
// draw_final_kernel walks those and re-reads one piece.
//
// The draw's weights are fp32 from the hardware exp2 for both logit types (fp32
// logits form the exponent in two parts to keep fp32-level accuracy), with fp64 sums
// across lanes and tiles; the merges of the streaming pass's records are fp64.
#include <type_traits>

#include "sv_draw.h"

namespace sv {

// ===========================================================================
// prepare: packed offsets of a ragged batch and the per-vector table
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
            // the row's vectors (bounds-checked: the totals are validated below), 8 at a
            // time with their token loads issued together before the stores
            const float T = P.temperature[i];
            for (int64_t k0 = 0; k0 <= g && t_off + k0 < P.nT; k0 += 8) {
                int32_t x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t k = k0 + j;
                    x[j] = (k < g && d_off + k < P.nD) ? P.tokens[d_off + k] : -1;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t k = k0 + j;
                    if (k > g || t_off + k >= P.nT) break;
                    const bool has_x = k < g && d_off + k < P.nD;
                    const int32_t slot = has_x ? (int32_t)(d_off + k) : -1;
                    P.vinfo[t_off + k] = VecInfo{(int32_t)i, slot, x[j], T};
                    if (P.mode == 0 && has_x) P.vinfo[P.nT + d_off + k] = VecInfo{(int32_t)i, slot, x[j], T};
                }
            }
        }
        __syncthreads();
        if (tid == 1023) { carry_t = pt + it; carry_d = pd + id; }
        __syncthreads();
    }
    if (tid == 0) P.hdr->status = (bad || carry_t != P.nT) ? ST_BAD_GAMMA : 0;
}

// ===========================================================================
// accept scan: the whole workgroup merges records, one wave tests positions
// ===========================================================================
constexpr int kScanBatch = 3;   // vectors per wave with their record loads in flight together

struct ScanLds {
    float m[2][64];        // per position of the chunk: target, draft maximum
    double S[2][64];       // sums 2^((z - m) c)
    int32_t idx[64];       // target first argmax (greedy rows)
    RowDraw D;
};

// One wave's record loads for vectors q0, q0 + 4, ... of a position chunk (vectors
// q < nt are target positions base + q, the others draft positions base + q - nt).
struct ScanBatch {
    Partial rec[kScanBatch];
    int64_t i0[kScanBatch], i1[kScanBatch];
};

template <int NW>
__device__ __forceinline__ void load_batch(const Params &P, const RowGeom &G, int64_t base, int nt, int nq, int q0,
                                           int lane, ScanBatch &B)
{
#pragma unroll
    for (int b = 0; b < kScanBatch; ++b) {
        const int q = q0 + b * NW;
        B.rec[b] = Partial{-INFINITY, INT32_MAX, 0.0};
        B.i0[b] = 0;
        B.i1[b] = -1;
        if (q < nq) {
            const int64_t v = q < nt ? G.t_off + base + q : P.nT + G.d_off + base + (q - nt);
            vec_records(P, v, B.i0[b], B.i1[b]);
            if (B.i0[b] + lane <= B.i1[b]) B.rec[b] = P.parts[B.i0[b] + lane];
        }
    }
}

// Per-vector statistics of positions [base, base + nt) (target) and [base, base + nd)
// (draft) of a row into LDS, each of the NW waves taking every NW-th vector (first:
// this wave's first batch, already loaded).  maxonly: every vector's records hold only
// a maximum (a row whose temperature is unusable).
template <int DT, int NW>
__device__ __forceinline__ void scan_merge(const Params &P, const RowGeom &G, int64_t base, int nt, int nd,
                                           bool greedy, const TempConst &tc, ScanLds &sh, const ScanBatch &first,
                                           bool have_first, bool maxonly)
{
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nq = nt + nd;
    for (int q0 = wave; q0 < nq; q0 += NW * kScanBatch) {
        ScanBatch B;
        if (have_first && q0 == wave) B = first;
        else load_batch<NW>(P, G, base, nt, nq, q0, lane, B);
#pragma unroll
        for (int b = 0; b < kScanBatch; ++b) {
            const int q = q0 + b * NW;
            if (q >= nq) break;
            float M;
            double S;
            int32_t idx;
            wave_merge<DT>(P, B.rec[b], B.i0[b], B.i1[b], (greedy && q < nt) || maxonly, tc, lane, M, S, idx);
            if (lane == 0) {
                const int side = q < nt ? 0 : 1, j = q < nt ? q : q - nt;
                sh.m[side][j] = M;
                sh.S[side][j] = S;
                if (side == 0) sh.idx[j] = idx;
            }

        }
    }
}

// Every output of an invalid row (one wave): nothing emitted, no diagnostics, no draw.
__device__ void ee_invalid_row(const Params &P, int32_t row, const RowGeom &G, int status, int lane)
{
    const int32_t g = G.gamma;
    for (int32_t k = lane; k <= g; k += 64) P.emitted[G.t_off + k] = -1;
    for (int32_t k = lane; k < g; k += 64) {
        if (P.p_x) P.p_x[G.d_off + k] = kQNaN;
        if (P.q_x) P.q_x[G.d_off + k] = kQNaN;
    }
    if (lane == 0) {
        P.n_accepted[row] = -1;
        if (P.row_status) P.row_status[row] = status;
        if (P.resid) P.resid[row] = kQNaN;
        if (P.crop_len) P.crop_len[row] = -1;
        P.draws[row].kind = DRAW_NONE;
    }
}

// The accept scan of one row by the whole workgroup of NW waves.  Returns what the draw
// needs (on every thread); with `write`, wave 0 also stores the row's outputs.
//
// EE: what the round with early exit sees, from a pass that read every position.  A
// row longer than that round's bound (gamma_max) is invalid outright.  A bad token
// anywhere makes a row invalid from the start; such a row, like one with an unusable
// temperature, still reports non-finite logits at any position.  Any other row counts
// status bits, and reports p(x_j), q(x_j), only up to its first rejection.
template <int DT, int NW = kWaves, bool EE = false>
__device__ RowDraw scan_row(const Params &P, int32_t row, bool write, ScanLds &sh)
{
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const RowGeom G = row_geom(P, row);
    const int32_t g = G.gamma;
    // every load that does not depend on the temperature first: the temperature, the
    // draw's uniform, the first position chunk's tokens, uniforms and logits at the
    // tokens (wave 0), and each wave's first batch of records
    const float T = P.temperature[row];
    const float u_draw = P.uniforms[G.t_off + g];
    int32_t x0 = 0;
    float u0 = 0.0f, zt0 = 0.0f, zd0 = 0.0f;
    if (wave == 0 && lane < g) {
        x0 = P.tokens[G.d_off + lane];
        u0 = P.uniforms[G.t_off + lane];
        if (P.mode == 0) {
            zt0 = P.zx[G.d_off + lane];
            zd0 = P.zx[P.nD + G.d_off + lane];
        }
    }
    ScanBatch first;
    {
        const int nt0 = g + 1 < 64 ? g + 1 : 64;
        const int nd0 = P.mode == 1 ? 0 : (g < 64 ? g : 64);
        load_batch<NW>(P, G, 0, nt0, nt0 + nd0, wave, lane, first);
    }
    const int32_t rm = row_mode(P.mode, T);
    const bool greedy = rm == ROW_GREEDY;
    const TempConst tc = temp_const<DT>(rm == ROW_SAMPLE ? T : 1.0f);
    int status = (rm == ROW_BAD_TEMP) ? ST_BAD_TEMP : 0;
    int32_t K = g;
    bool found = false;
    float kmt = -INFINITY, kmd = -INFINITY;   // statistics at K (wave 0, every lane once known)
    double kSt = 0.0, kSd = 0.0;
    int32_t kidx = -1;
    int32_t x_keep = 0;                       // this lane's draft token (rows with gamma < 64)

    // a row with an unusable temperature decides nothing, but every position is still
    // checked for non-finite logits (from the maxima its records hold)
    const bool bad = rm == ROW_BAD_TEMP;
    bool pre_invalid = bad;   // (wave 0)
    if constexpr (EE) {
        if (g > P.gamma_max) {
            if (write && wave == 0) ee_invalid_row(P, row, G, ST_BAD_GAMMA, lane);
            RowDraw D{};
            D.kind = DRAW_NONE;
            return D;
        }
        if (wave == 0) {
            int badx = 0;
            for (int32_t k = lane; k < g; k += 64) {
                const int32_t xk = k < 64 ? x0 : P.tokens[G.d_off + k];
                if (xk < 0 || (int64_t)xk >= P.V) badx = 1;
            }
            if (wave_or_int(badx)) pre_invalid = true;
        }
    }
    {
        for (int64_t base = 0; base <= g; base += 64) {
            const int nt = (int)(g + 1 - base < 64 ? g + 1 - base : 64);
            const int nd = greedy ? 0 : (int)(g - base < 64 ? g - base : 64);
            const int64_t j = base + lane;
            const bool has_t = j <= g, has_d = j < g;
            // this chunk's per-position inputs (wave 0), in flight during the merge
            int32_t x = x0;
            float u = u0, zt = zt0, zd = zd0;
            if (base > 0 && wave == 0 && has_d) {
                x = P.tokens[G.d_off + j];
                u = P.uniforms[G.t_off + j];
                if (!greedy) {
                    zt = P.zx[G.d_off + j];
                    zd = P.zx[P.nD + G.d_off + j];
                }
            }
            scan_merge<DT, NW>(P, G, base, nt, nd, greedy, tc, sh, first, base == 0, bad);
            __syncthreads();
            if (wave == 0) {
                x_keep = x;
                const bool x_ok = x >= 0 && (int64_t)x < P.V;
                int cs = 0;   // this lane's status bits at position j
                if (has_d && !x_ok) cs |= ST_BAD_TOKEN;
                const float mt = has_t ? sh.m[0][lane] : -INFINITY;
                const double St = has_t ? sh.S[0][lane] : 0.0;
                const int32_t it = has_t ? sh.idx[lane] : INT32_MAX;
                float md = -INFINITY;
                double Sd = 0.0;
                double px = kQNaN, qx = kQNaN;
                bool reject = false;
                if (bad) {
                    if (has_t && !(mt > -INFINITY && mt < INFINITY)) cs |= ST_NONFINITE;
                    if (has_d && !(sh.m[1][lane] > -INFINITY && sh.m[1][lane] < INFINITY)) cs |= ST_NONFINITE;
                } else if (greedy) {
                    if (has_t && !(mt > -INFINITY && mt < INFINITY)) cs |= ST_NONFINITE;
                    if (has_d) reject = x != it;
                } else {
                    if (has_t && !(St > 0.0 && St < INFINITY)) cs |= ST_NONFINITE;
                    if (has_d) {
                        md = sh.m[1][lane];
                        Sd = sh.S[1][lane];
                        if (!(Sd > 0.0 && Sd < INFINITY)) cs |= ST_NONFINITE;
                        if (x_ok && St > 0.0 && St < INFINITY && Sd > 0.0 && Sd < INFINITY) {
                            px = exp2_f64(((double)zt - (double)mt) * tc.c_eff) / St;
                            qx = exp2_f64(((double)zd - (double)md) * tc.c_eff) / Sd;
                            double ratio;
                            if (qx > 0.0) {
                                ratio = px / qx;
                                if (ratio > 1.0) ratio = 1.0;
                            } else {
                                ratio = px > 0.0 ? 1.0 : 0.0;
                                cs |= ST_Q_ZERO;
                            }
                            reject = !((double)u < ratio);
                        }
                    }
                }
                const bool was_found = found;
                const unsigned long long rb = __ballot(reject);
                int src = -1;
                if (!found && rb != 0ull) {
                    src = __ffsll((long long)rb) - 1;
                    K = (int32_t)(base + src);
                    found = true;
                } else if (!found && g - base < 64) {
                    src = (int)(g - base);   // no rejection: the bonus position is in this chunk
                }
                // the positions that count: all of them, or (early exit) those up to the
                // first rejection
                bool counts = true;
                if constexpr (EE) counts = pre_invalid || (!was_found && (!found || (int64_t)lane <= K - base));
                if (counts) status |= cs;
                if (write && has_d && !bad && !greedy) {
                    if (P.p_x) P.p_x[G.d_off + j] = counts ? px : kQNaN;
                    if (P.q_x) P.q_x[G.d_off + j] = counts ? qx : kQNaN;
                }
                if (src >= 0) {
                    kmt = __shfl(mt, src);
                    kSt = __shfl(St, src);
                    kmd = __shfl(md, src);
                    kSd = __shfl(Sd, src);
                    kidx = __shfl(it, src);
                }
            }
            // every chunk is scanned (statuses and diagnostics cover all positions)
            __syncthreads();   // sh is rewritten by the next chunk
        }
    }

    if (wave == 0) {
        status = wave_or_int(status);
        const bool invalid = (status & ST_INVALID) != 0;
        if (invalid) status &= ST_INVALID;   // an invalid row makes no decision to describe
        RowDraw D{};
        D.kind = DRAW_NONE;
        if (!invalid && !greedy) {
            D.kind = K < g ? DRAW_RESIDUAL : DRAW_BONUS;
            D.K = K;
            D.t_row = (int32_t)(G.t_off + K);
            D.d_row = (int32_t)(G.d_off + K);
            D.u = u_draw;
            D.t_slot = (int32_t)(G.t_off + K);
            D.m_t = kmt;
            D.S_t = kSt;
            D.m_d = kmd;
            D.S_d = kSd;
            D.T = T;
            D.theta_t = P.theta ? P.theta[D.t_row] : -INFINITY;
            D.theta_d = (P.theta && K < g) ? P.theta[P.nT + D.d_row] : -INFINITY;
        }
        if (write) {
            for (int64_t j = lane; j <= g; j += 64) {
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
                if (P.crop_len)
                    P.crop_len[row] = invalid ? -1 : (int32_t)((P.cache_len ? P.cache_len[row] : 0) + K + 1);
                P.draws[row] = D;
            }
        }
        if (lane == 0) sh.D = D;
    }
    __syncthreads();
    return sh.D;
}

// Ragged batch whose gamma array is inconsistent: every row and slot is invalid (NT:
// the workgroup's threads).
template <int NT>
__device__ void invalidate_call(const Params &P, int32_t row, bool row_writer)
{
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * NT;
    for (int64_t s = gid; s < P.nT; s += nthreads) P.emitted[s] = -1;
    for (int64_t s = gid; s < P.nD; s += nthreads) {
        if (P.p_x) P.p_x[s] = kQNaN;
        if (P.q_x) P.q_x[s] = kQNaN;
    }
    if (row_writer && row < P.B) {
        P.n_accepted[row] = -1;
        if (P.row_status) P.row_status[row] = ST_BAD_GAMMA;
        if (P.resid) P.resid[row] = kQNaN;
        if (P.crop_len) P.crop_len[row] = -1;
        P.draws[row].kind = DRAW_NONE;
    }
}

// ===========================================================================
// early exit: the positions of each row left to right, in chunks
// ===========================================================================
// Step k reads positions [2^k - 1, 2^(k+1) - 1) of the rows still undecided (the
// vectors of the whole chunk in one streaming launch) and then decides them in order,
// stopping at the first rejection: the first step reads position 0 of every row, and
// a row that keeps accepting takes a step per doubling of its accepted length.

// The first lists: every row, with its position-0 vectors (target in slot i, draft in
// slot B + i or -1); every output slot starts invalid (-1, NaN) and is filled as the
// steps decide.
__global__ __launch_bounds__(kBlock) void ee_init_kernel(Params P)
{
    const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * kBlock;
    const bool bad_call = P.gamma != nullptr && P.hdr->status != 0;
    if (gid == 0) {
        const bool sample = P.mode == 0;
        P.ee_count[0] = bad_call ? 0 : P.B;
        P.ee_count[1] = bad_call ? 0 : (sample ? 2 * P.B : P.B);
        P.ee_count[2] = 0;
        P.ee_count[3] = 0;
    }
    if (bad_call) {
        for (int64_t s = gid; s < P.nT; s += nth) P.emitted[s] = -1;
        for (int64_t s = gid; s < P.nD; s += nth) {
            if (P.p_x) P.p_x[s] = kQNaN;
            if (P.q_x) P.q_x[s] = kQNaN;
        }
    }
    for (int64_t i = gid; i < P.B; i += nth) {
        P.draws[i].kind = DRAW_NONE;
        if (bad_call) {
            P.n_accepted[i] = -1;
            if (P.row_status) P.row_status[i] = ST_BAD_GAMMA;
            if (P.resid) P.resid[i] = kQNaN;
            if (P.crop_len) P.crop_len[i] = -1;
            continue;
        }
        const RowGeom G = row_geom(P, (int32_t)i);
        const int32_t g = G.gamma;
        // a row longer than the bound the steps cover is invalid and reads nothing
        const bool over = g > P.gamma_max;
        P.ee_status[i] = over ? ST_BAD_GAMMA : 0;
        P.ee_rows[0][i] = (int32_t)i;
        P.ee_vecs[0][i] = over ? -1 : (int32_t)G.t_off;
        if (P.mode == 0) P.ee_vecs[0][P.B + i] = (!over && g > 0) ? (int32_t)(P.nT + G.d_off) : -1;
        for (int32_t k = 0; k <= g; ++k) P.emitted[G.t_off + k] = -1;
        for (int32_t k = 0; k < g; ++k) {
            if (P.p_x) P.p_x[G.d_off + k] = kQNaN;
            if (P.q_x) P.q_x[G.d_off + k] = kQNaN;
        }
        if (P.resid) P.resid[i] = kQNaN;
        if (over) {
            P.n_accepted[i] = -1;
            if (P.row_status) P.row_status[i] = ST_BAD_GAMMA;
            if (P.crop_len) P.crop_len[i] = -1;
        }
    }
}

// One workgroup per listed row decides the positions of this step's chunk: its waves
// merge the records of every vector of the chunk together, then wave 0 tests all the
// positions at once (lane i: position j0 + i) and takes the first event, in position
// order: non-finite logits (the row is invalid), the rejection of draft j (or its
// argmax mismatch), or the bonus at j = gamma.  Positions before it are kept.  A row
// invalid from the start (a bad temperature or token) has no event but non-finite
// logits and its last position.  A row with no event in the chunk is listed for the
// next chunk, with that chunk's vectors.
constexpr int kEeWaves = 4;

template <int DT>
__global__ __launch_bounds__(kEeWaves * 64) void ee_step_kernel(Params P)
{
    __shared__ ScanLds sh;
    __shared__ int s_stop;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int buf = P.step & 1;
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    // the row id is read together with the count (slot < B, so in the list's buffer),
    // one dependent read fewer before the row's own
    const int32_t slot = (int32_t)blockIdx.x;
    const int32_t listed = P.ee_count[2 * buf];
    const int32_t row = P.ee_rows[buf][slot];
    if (slot >= listed) return;
    int status = P.ee_status[row];
    if (status & ST_BAD_GAMMA) return;   // invalid from the start, outputs already written
    const RowGeom G = row_geom(P, row);
    const int32_t g = G.gamma;
    const int32_t j0 = P.ee_j0, j1 = P.ee_j1 <= g ? P.ee_j1 : g + 1;   // this step's positions
    const float T = P.temperature[row];
    const float u_draw = P.uniforms[G.t_off + g];
    const int32_t rm = row_mode(P.mode, T);
    const bool greedy = rm == ROW_GREEDY, maxonly = rm == ROW_BAD_TEMP;
    const int64_t n_cache = P.cache_len ? P.cache_len[row] : 0;
    if (j0 == 0 && wave == 0) {
        if (rm == ROW_BAD_TEMP) status |= ST_BAD_TEMP;
        int bad = 0;
        for (int32_t k = lane; k < g; k += 64) {
            const int32_t xk = P.tokens[G.d_off + k];
            if (xk < 0 || (int64_t)xk >= P.V) bad = 1;
        }
        if (wave_or_int(bad)) status |= ST_BAD_TOKEN;
    }
    const bool pre_invalid = (status & (ST_BAD_TEMP | ST_BAD_TOKEN)) != 0;   // read on wave 0 only
    const TempConst tc = temp_const<DT>(rm == ROW_SAMPLE ? T : 1.0f);
    ScanBatch none;
    for (int32_t base = j0; base < j1; base += 64) {
        const int nt = j1 - base < 64 ? j1 - base : 64;
        const int32_t dend = j1 < g ? j1 : g;
        const int nd = greedy || dend <= base ? 0 : (dend - base < 64 ? dend - base : 64);
        // wave 0: this sub-chunk's per-position inputs, in flight during the merge
        const int32_t j = base + lane;
        const bool in = lane < nt, has_d = in && j < g;
        int32_t x = -1;
        float u = 0.0f, zt = 0.0f, zd = 0.0f;
        if (wave == 0 && has_d) {
            x = P.tokens[G.d_off + j];
            u = P.uniforms[G.t_off + j];
            if (!greedy) {
                zt = P.zx[G.d_off + j];
                zd = P.zx[P.nD + G.d_off + j];
            }
        }
        scan_merge<DT, kEeWaves>(P, G, base, nt, nd, greedy, tc, sh, none, false, maxonly);
        __syncthreads();
        if (wave == 0) {
            const float mt = in ? sh.m[0][lane] : -INFINITY;
            const double St = in ? sh.S[0][lane] : 0.0;
            const int32_t at = in ? sh.idx[lane] : INT32_MAX;
            const float md = has_d && !greedy ? sh.m[1][lane] : -INFINITY;
            const double Sd = has_d && !greedy ? sh.S[1][lane] : 0.0;
            bool nonfinite = false, reject = false, qzero = false;
            double px = kQNaN, qx = kQNaN;
            if (in) {
                nonfinite = (greedy || maxonly) ? !(mt > -INFINITY && mt < INFINITY) : !(St > 0.0 && St < INFINITY);
                if (has_d && !greedy)
                    nonfinite |= maxonly ? !(md > -INFINITY && md < INFINITY) : !(Sd > 0.0 && Sd < INFINITY);
            }
            if (in && !nonfinite && !pre_invalid && has_d) {
                if (greedy) {
                    reject = x != at;
                } else {
                    px = exp2_f64(((double)zt - (double)mt) * tc.c_eff) / St;
                    qx = exp2_f64(((double)zd - (double)md) * tc.c_eff) / Sd;
                    double ratio;
                    if (qx > 0.0) {
                        ratio = px / qx;
                        if (ratio > 1.0) ratio = 1.0;
                    } else {
                        ratio = px > 0.0 ? 1.0 : 0.0;
                        qzero = true;
                    }
                    reject = !((double)u < ratio);
                }
            }
            const bool event = in && (nonfinite || j == g || reject);
            const unsigned long long eb = __ballot(event);
            const int e = eb ? __ffsll((long long)eb) - 1 : 64;   // first event's lane
            status |= wave_or_int(lane <= e && qzero ? ST_Q_ZERO : 0);
            const bool nf = e < 64 && __shfl(nonfinite ? 1 : 0, e) != 0;
            if (e < 64 && (nf || pre_invalid)) {
                if (nf) status |= ST_NONFINITE;
                for (int32_t k = lane; k <= g; k += 64) P.emitted[G.t_off + k] = -1;
                for (int32_t k = lane; k < g; k += 64) {
                    if (P.p_x) P.p_x[G.d_off + k] = kQNaN;
                    if (P.q_x) P.q_x[G.d_off + k] = kQNaN;
                }
                if (lane == 0) {
                    P.n_accepted[row] = -1;
                    if (P.row_status) P.row_status[row] = status & ST_INVALID;
                    if (P.resid) P.resid[row] = kQNaN;
                    if (P.crop_len) P.crop_len[row] = -1;
                }
            } else if (!pre_invalid) {
                // positions before the event are kept; at the event a greedy row emits the
                // argmax, a sampling row's token is drawn later
                if (lane < e && in) P.emitted[G.t_off + j] = x;
                if (greedy && lane == e) P.emitted[G.t_off + j] = at;
                if (!greedy && lane <= e && has_d) {
                    if (P.p_x) P.p_x[G.d_off + j] = px;
                    if (P.q_x) P.q_x[G.d_off + j] = qx;
                }
                if (e < 64) {
                    const int32_t K = base + e;
                    RowDraw D{};
                    D.kind = greedy ? DRAW_NONE : (K < g ? DRAW_RESIDUAL : DRAW_BONUS);
                    const float kmt = __shfl(mt, e), kmd = __shfl(md, e);
                    const double kSt = __shfl(St, e), kSd = __shfl(Sd, e);
                    if (D.kind != DRAW_NONE) {
                        D.K = K;
                        D.t_row = (int32_t)(G.t_off + K);
                        D.d_row = (int32_t)(G.d_off + K);
                        D.u = u_draw;
                        D.t_slot = (int32_t)(G.t_off + K);
                        D.m_t = kmt;
                        D.S_t = kSt;
                        D.m_d = kmd;
                        D.S_d = kSd;
                        D.T = T;
                        D.theta_t = -INFINITY;
                        D.theta_d = -INFINITY;
                    }
                    if (lane == 0) {
                        P.n_accepted[row] = K;
                        if (P.row_status) P.row_status[row] = status;
                        if (P.crop_len) P.crop_len[row] = (int32_t)(n_cache + K + 1);
                        P.draws[row] = D;
                    }
                }
            }
            if (lane == 0) s_stop = e < 64 ? 1 : 0;
        }
        __syncthreads();
        if (s_stop) return;
    }
    if (wave != 0) return;
    // no event through the chunk (j1 <= g here): listed for the next chunk, positions
    // [j1, min(ee_j2, g + 1)), with their target vectors, then their draft vectors
    const int32_t a = j1, b = P.ee_j2 <= g ? P.ee_j2 : g + 1;
    const int32_t nt = b - a, nd = greedy ? 0 : (b <= g ? b : g) - a;
    int32_t base = 0;
    if (lane == 0) {
        P.ee_status[row] = status;
        const int32_t s2 = atomicAdd(&P.ee_count[2 * (buf ^ 1)], 1);
        base = atomicAdd(&P.ee_count[2 * (buf ^ 1) + 1], nt + nd);
        P.ee_rows[buf ^ 1][s2] = row;
    }
    base = __shfl(base, 0);
    for (int32_t q = lane; q < nt + nd; q += 64)
        P.ee_vecs[buf ^ 1][base + q] = q < nt ? (int32_t)(G.t_off + a + q) : (int32_t)(P.nT + G.d_off + a + (q - nt));
}

// ===========================================================================
// draw: per-tile weight sums, then the inverse CDF
// ===========================================================================
// The accept scan, one workgroup per row; it stores the row's outputs and what the
// draw needs.
template <int DT, bool EE>
__device__ __forceinline__ void scan_body(const Params &P)
{
    __shared__ ScanLds sh;
    const int32_t row = (int32_t)blockIdx.x;
    if (P.gamma != nullptr && P.hdr->status != 0) {
        invalidate_call<kBlock>(P, row, threadIdx.x == 0);
        return;
    }
    scan_row<DT, kWaves, EE>(P, row, true, sh);
}

// EE: the decisions of the round with early exit (see scan_row)
template <int DT, bool EE>
__global__ __launch_bounds__(kBlock) void scan_kernel(Params P)
{
    scan_body<DT, EE>(P);
}

// Sums of the draw weights w (the residual max(0, p - q), or p) and of p over the NTW
// tiles t0 .. t0 + NTW - 1 of the row's position K, all their loads in flight together;
// tiles at or past t_end add nothing and are not stored.
template <int DT, bool AL, int NTW>
__device__ __forceinline__ void tile_sums(const Params &P, const DrawConst<DT> &c, const RowDraw &D, int32_t row,
                                          int64_t t0, int64_t t_end, int lane)
{
    const void *tb = vec_ptr(P.target, DT, D.t_row, P.V);
    const void *db = c.residual ? vec_ptr(P.draft, DT, D.d_row, P.V) : nullptr;
    RawUnit<DT> rt[NTW], rd[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int64_t unit = (t0 + i) * kTileUnits + lane;
        const bool in = t0 + i < t_end && unit < P.geo.nunits;
        if constexpr (AL) {
            rt[i] = in ? load_raw<DT, AL>(tb, unit, P.V) : neg_inf_unit<DT>();
            rd[i] = (in && c.residual) ? load_raw<DT, AL>(db, unit, P.V) : neg_inf_unit<DT>();
        } else {
            rt[i] = load_tile_unit<DT>(tb, t0 + i, P.V, P.target, array_bytes(P, DT, true), lane);
            rd[i] = c.residual ? load_tile_unit<DT>(db, t0 + i, P.V, P.draft, array_bytes(P, DT, false), lane)
                               : neg_inf_unit<DT>();
        }
    }
    // per-lane sums of every tile first, then one cross-lane reduction of all of them
    // (tiles past the end read -inf logits and sum to 0)
    constexpr int NV = 2 * NTW;   // w and p of each tile: value 2 i + 1 is tile i's p
    static_assert(NV >= 2 && NV <= 64 && (NV & (NV - 1)) == 0, "tile batch");
    double v[NV];
    // A lane's 8 terms of a tile summed in fp32 (bf16: in order and without their
    // common factor 1 / S_t, relative error at most 7 units of 2^-24; fp32 logits:
    // pairwise, at most 3 units, within the 1e-6 to which their residual mass is
    // held; both well below the 1e-5 W at which a draw counts as near), the
    // comparisons with the thresholds only in filtered calls and the kind of draw
    // fixed per variant (straight-line code): the reduction is bound by its
    // arithmetic once the loads are in.
    static_assert(kUnitElems == 8, "unit of 8 logits");
    auto units = [&](auto filt, auto res) {
        constexpr bool F = decltype(filt)::value;
        constexpr int R = decltype(res)::value;
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            float zt[kUnitElems], zd[kUnitElems], sw, sp;
            unpack<DT>(rt[i], zt);
            unpack<DT>(rd[i], zd);
            if constexpr (DT == 0) {
                c.template unit_sums<F, R>(zt, zd, sw, sp);
            } else {
                float w[kUnitElems], p[kUnitElems];
                c.template weights<F, R>(zt, zd, w, p);
                sw = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
                sp = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            }
            v[2 * i] = sw;
            v[2 * i + 1] = sp;
        }
    };
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    if (c.filt) {
        if (c.residual) units(std::true_type{}, R1{});
        else units(std::true_type{}, R0{});
    } else {
        if (c.residual) units(std::false_type{}, R1{});
        else units(std::false_type{}, R0{});
    }
    double scale = 1.0;
    if constexpr (DT == 0) scale = c.Ftd;
    // Reduce-scatter over the wave: each exchange halves the values a lane holds (the
    // lane whose bit o is set keeps the upper half and sends the lower), so after
    // log2 NV exchanges lane l holds a partial sum of value l >> (6 - log2 NV); the
    // remaining exchanges sum that one value over the lanes that share it.
#pragma unroll
    for (int n = NV, o = 32; n > 1; n >>= 1, o >>= 1) {
        const bool hi = (lane & o) != 0;
#pragma unroll
        for (int k = 0; k < n / 2; ++k) {
            const double keep = hi ? v[k + n / 2] : v[k];
            const double send = hi ? v[k] : v[k + n / 2];
            v[k] = keep + __shfl_xor(send, o);
        }
    }
    constexpr int kGroup = 64 / NV;   // lanes that hold one value
#pragma unroll
    for (int o = kGroup / 2; o > 0; o >>= 1) v[0] += __shfl_xor(v[0], o);
    if ((lane & (kGroup - 1)) == 0) {
        const int idx = lane / kGroup, i = idx >> 1;
        if (t0 + i < t_end) {
            Sum2 *d = &P.tiles[row * P.geo.ntiles + t0 + i];
            *((idx & 1) ? &d->p : &d->w) = v[0] * scale;
        }
    }
}

// The residual's tile sums: workgroup `piece` of a row that rejected sums its slice of
// position K.
template <int DT, bool AL>
__device__ __forceinline__ void verify_body(const Params &P)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t per_row = (uint32_t)P.geo.ndraw;
    const int32_t row = (int32_t)(blockIdx.x / per_row);
    const int32_t piece = (int32_t)(blockIdx.x - (uint32_t)row * per_row);
    const RowDraw D = P.draws[row];   // loaded together with the status word
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    // bonus draws use the streaming pass's piece sums, except when p is filtered
    if (!(D.kind == DRAW_RESIDUAL || (P.theta && D.kind == DRAW_BONUS))) return;
    DrawConst<DT> c;
    c.init(D);
    const int64_t t0 = (int64_t)piece * kTilesPerDrawWg + (int64_t)wave * kTilesPerWave;
    tile_sums<DT, AL, kTilesPerWave>(P, c, D, row, t0, P.geo.ntiles, lane);
}

// The accept scan and the residual's tile sums in one kernel: st_split workgroups of 16
// waves per row.  Each runs the row's scan (the same arithmetic in each, so the same K
// and draw record), the first also writes the row's outputs, and each then sums the
// residual over its share of the row's tiles at position K, with no round trip through
// memory between the decision and the loads of position K.
constexpr int kScanTileBlock = 1024;
constexpr int kScanTileWaves = kScanTileBlock / 64;
constexpr int kScanTileBatch = 4;   // tiles per wave with all their loads in flight

template <int DT, bool AL, bool EE>
__device__ __forceinline__ void scan_tiles_body(const Params &P)
{
    __shared__ ScanLds sh;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t S = (uint32_t)P.st_split;   // (32-bit: a 64-bit division costs ~100 instructions)
    const int32_t row = (int32_t)(blockIdx.x / S);
    const int32_t part = (int32_t)(blockIdx.x - (uint32_t)row * S);
    if (P.gamma != nullptr && P.hdr->status != 0) {
        invalidate_call<kScanTileBlock>(P, row, part == 0 && threadIdx.x == 0);
        return;
    }
    const RowDraw D = scan_row<DT, kScanTileWaves, EE>(P, row, part == 0, sh);
    // bonus draws use the streaming pass's piece sums, except when p is filtered
    if (!(D.kind == DRAW_RESIDUAL || (P.theta && D.kind == DRAW_BONUS))) return;
    DrawConst<DT> c;
    c.init(D);
    const uint32_t nt = (uint32_t)P.geo.ntiles;   // (nt S < 2^32: 32-bit divisions)
    const int64_t a = nt * (uint32_t)part / S, b = nt * (uint32_t)(part + 1) / S;
    for (int64_t t0 = a + (int64_t)wave * kScanTileBatch; t0 < b; t0 += (int64_t)kScanTileWaves * kScanTileBatch)
        tile_sums<DT, AL, kScanTileBatch>(P, c, D, row, t0, b, lane);
}

template <int DT, bool AL, bool EE>
__global__ __launch_bounds__(kScanTileBlock) void scan_tiles_kernel(Params P)
{
    scan_tiles_body<DT, AL, EE>(P);
}

template <bool AL>
__global__ __launch_bounds__(kBlock) void verify_kernel(Params P)
{
    verify_body<0, AL>(P);
}

template <bool AL>
__global__ __launch_bounds__(kBlock) void verify_kernel_f32(Params P)
{
    verify_body<1, AL>(P);
}

// ---------------------------------------------------------------------------
// bonus draw from the streaming pass's records: the weights are p at position K, so
// the piece sums are already known (the sum 2^((z - M_j) c) of piece j, taken to the
// vector maximum m and divided by S).  One wave per row finds the piece where the
// running sum first exceeds t = u W, then re-reads that piece only: its tiles'
// sums, the tile, the token.
// ---------------------------------------------------------------------------

// The bonus draw by the workgroup's four waves: the piece (chosen by the scan, or
// here for vectors of more than 64 pieces), each wave's quarter of its tiles summed,
// the tile, the token.
template <int DT, bool AL>
__device__ __forceinline__ void draw_bonus_row(const Params &P, const RowDraw &D, int32_t row, int lane, int wave,
                                               double *s_ts)
{
    const TempConst tc = temp_const<DT>(D.T);
    int64_t piece = -1;
    double before = 0.0, W = 0.0;
    // the piece from the records (every wave computes the same): one per lane when the
    // vector has at most 64 pieces, else contiguous runs per lane
    if (P.geo.ipv <= 64) {
        const Partial q = lane < P.geo.ipv ? P.parts[(int64_t)D.t_row * P.geo.ipv + lane]
                                           : Partial{-INFINITY, INT32_MAX, 0.0};
        int32_t pc;
        bonus_piece<DT>(q, tc, D.m_t, D.S_t, D.u, lane, pc, before, W);
        piece = pc;
    } else {
        const int64_t ipv = P.geo.ipv;
        const Partial *rec = P.parts + (int64_t)D.t_row * ipv;
        const int64_t per = (ipv + 63) / 64;
        const int64_t l0 = lane * per;
        const int64_t l1 = min(l0 + per, ipv);
        double lw = 0.0;
        for (int64_t j = l0; j < l1; ++j) lw += piece_weight<DT>(rec[j], tc, D.m_t, D.S_t);
        const double iw = wave_inclusive_sum(lw, lane);
        W = __shfl(iw, 63);
        const double t = (double)D.u * W;
        double cum = iw - lw;
        int64_t cand = -1, lastpos = -1;
        double cand_before = 0.0, last_before = 0.0;
        for (int64_t j = l0; j < l1; ++j) {
            const double v = piece_weight<DT>(rec[j], tc, D.m_t, D.S_t);
            if (cand < 0 && cum + v > t) { cand = j; cand_before = cum; }
            if (v > 0.0) { lastpos = j; last_before = cum; }
            cum += v;
        }
        const unsigned long long hit = __ballot(cand >= 0);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            piece = __shfl(cand, l);
            before = __shfl(cand_before, l);
        } else {
            const unsigned long long pos = __ballot(lastpos >= 0);
            if (pos) {
                const int l = 63 - __clzll((long long)pos);
                piece = __shfl(lastpos, l);
                before = __shfl(last_before, l);
            }
        }
    }
    const double t = (double)D.u * W;
    constexpr int NT = kPieceTiles<DT>;
    constexpr int NW = NT / kWaves;   // tiles per wave
    if (piece < 0) {   // no piece has weight (cannot happen for a valid row)
        if (wave == 0 && lane == 0) {
            P.emitted[D.t_slot] = -1;
            if (P.resid) P.resid[row] = W;
        }
        return;
    }
    DrawConst<DT> c;
    c.init(D);
    const void *tb = vec_ptr(P.target, DT, D.t_row, P.V);
    const int64_t tile0 = piece * NT + wave * NW;
    RawUnit<DT> r[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const int64_t unit = (tile0 + k) * kTileUnits + lane;
        if constexpr (AL) r[k] = unit < P.geo.nunits ? load_raw<DT, AL>(tb, unit, P.V) : neg_inf_unit<DT>();
        else r[k] = load_tile_unit<DT>(tb, tile0 + k, P.V, P.target, array_bytes(P, DT, true), lane);
    }
    double ls[NW], ts[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        float z[kUnitElems];
        unpack<DT>(r[k], z);
        typename DrawConst<DT>::W w[kUnitElems], pe[kUnitElems];
        c.weights(z, z, w, pe);
        ls[k] = 0.0;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) ls[k] += pe[e];
        ts[k] = ls[k];
    }
    wave_totals<NW>(ts, lane);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < NW; ++k) s_ts[wave * NW + k] = ts[k];
    }
    __syncthreads();
    // the tile where the running sum first exceeds t, else the last tile of the piece
    // with weight (a crossing lost to rounding between the two sums)
    int kt = -1, kl = -1;
    double tb_hit = 0.0, tb_last = 0.0, run = before;
    for (int k = 0; k < NT; ++k) {
        const double v = s_ts[k];
        if (kt < 0 && run + v > t) { kt = k; tb_hit = run; }
        if (v > 0.0) { kl = k; tb_last = run; }
        run += v;
    }
    const int k_sel = kt >= 0 ? kt : kl;
    int32_t token = -1;
    if (k_sel >= 0 && k_sel / NW == wave) {
        const double tile_before = kt >= 0 ? tb_hit : tb_last;
        const int ks = k_sel - wave * NW;
        double my = 0.0;
        RawUnit<DT> rs = r[0];
#pragma unroll
        for (int k = 0; k < NW; ++k)
            if (k == ks) { my = ls[k]; rs = r[k]; }
        float z[kUnitElems];
        unpack<DT>(rs, z);
        typename DrawConst<DT>::W w[kUnitElems], pe[kUnitElems];
        c.weights(z, z, w, pe);
        const double incl = wave_inclusive_sum(my, lane);
        double rr = tile_before + incl - my;
        int ce = -1, lpos = -1;
#pragma unroll
        for (int e = 0; e < kUnitElems; ++e) {
            const double we = pe[e];
            rr += we;
            if (ce < 0 && rr > t) ce = e;
            if (we > 0.0) lpos = e;
        }
        const int64_t unit = (tile0 + ks) * kTileUnits + lane;
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
        // no logit of the piece has a weight in fp32 although its record does (its
        // probability is below 2^-126): the piece's first logit stands in
        if (token < 0) token = (int32_t)(piece * NT * kTileElems);
        if (lane == 0) {
            P.emitted[D.t_slot] = token;
            if (P.resid) P.resid[row] = W;
        }
    } else if (k_sel < 0 && wave == 0 && lane == 0) {
        P.emitted[D.t_slot] = (int32_t)(piece * NT * kTileElems);
        if (P.resid) P.resid[row] = W;
    }
}

// A lane's tile sums of the residual walk, R at a time with all R loads in flight
// together (one round trip for vocabularies up to 64 R tiles); the lane holds the
// contiguous tiles [l0, l1) of its row, and tiles past l1 read as 0.
constexpr int kWalkChunk = 8;
struct TileChunk {
    double w[kWalkChunk], p[kWalkChunk];
};

__device__ __forceinline__ void walk_range(const Params &P, int lane, int &per, int &l0, int &l1)
{
    const int32_t nt = P.geo.ntiles;
    per = (nt + 63) / 64;
    l0 = lane * per;
    l1 = min(l0 + per, nt);
}

__device__ __forceinline__ void load_tile_chunk(const Sum2 *tiles, int c0, int l1, TileChunk &c)
{
#pragma unroll
    for (int i = 0; i < kWalkChunk; ++i) {
        const Sum2 x = c0 + i < l1 ? tiles[c0 + i] : Sum2{0.0, 0.0};
        c.w[i] = x.w;
        c.p[i] = x.p;
    }
}

// The residual draw from the tile sums of the row's position K; `ch` holds the lane's
// first chunk of them (load_tile_chunk at l0).
template <int DT, bool AL>
__device__ __forceinline__ void draw_residual_row(const Params &P, const RowDraw &D, int32_t row, int lane,
                                                  TileChunk &ch)
{
    const Sum2 *tiles = P.tiles + (int64_t)row * P.geo.ntiles;
    int per, l0, l1;
    walk_range(P, lane, per, l0, l1);
    constexpr int R = kWalkChunk;
    double *rw = ch.w, *rp = ch.p;

    // total weight (residual, or p when the residual is empty)
    double lw = 0.0, lp = 0.0;
    for (int c0 = l0; c0 < l1; c0 += R) {
        if (c0 != l0) load_tile_chunk(tiles, c0, l1, ch);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            lw += rw[i];
            lp += rp[i];
        }
    }
    const double iw = wave_inclusive_sum(lw, lane), ip = wave_inclusive_sum(lp, lane);
    double W = __shfl(iw, 63);
    bool use_p = false;
    if (D.kind == DRAW_RESIDUAL && !(W > 0.0)) use_p = true;
    if (use_p) W = __shfl(ip, 63);
    const double t = (double)D.u * W;

    // the tile where the running sum first exceeds t
    double cum = use_p ? ip - lp : iw - lw;
    int cand = -1, lastpos = -1;
    double cand_before = 0.0, last_before = 0.0;
    for (int c0 = l0; c0 < l1; c0 += R) {
        if (per > R) load_tile_chunk(tiles, c0, l1, ch);   // (else ch still holds the lane's tiles)
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int k = c0 + i;
            if (k >= l1) break;
            const double v = use_p ? rp[i] : rw[i];
            if (cand < 0 && cum + v > t) { cand = k; cand_before = cum; }
            if (v > 0.0) { lastpos = k; last_before = cum; }
            cum += v;
        }
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
        RawUnit<DT> rt, rd;
        if constexpr (AL) {
            rt = in ? load_raw<DT, AL>(tb, unit, P.V) : neg_inf_unit<DT>();
            rd = (in && c.residual) ? load_raw<DT, AL>(db, unit, P.V) : neg_inf_unit<DT>();
        } else {
            rt = load_tile_unit<DT>(tb, tile, P.V, P.target, array_bytes(P, DT, true), lane);
            rd = c.residual ? load_tile_unit<DT>(db, tile, P.V, P.draft, array_bytes(P, DT, false), lane)
                            : neg_inf_unit<DT>();
        }
        float zt[kUnitElems], zd[kUnitElems];
        unpack<DT>(rt, zt);
        unpack<DT>(rd, zd);
        typename DrawConst<DT>::W w[kUnitElems], p[kUnitElems];
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

// One workgroup of four waves per row: the residual walk runs on wave 0, the bonus
// draw on all four.
template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void draw_final_kernel(Params P)
{
    __shared__ double s_ts[kPieceTiles<DT>];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t row = blockIdx.x;
    // the residual walk's first tile sums need only the row: their loads overlap the
    // draw record's (for rows that draw otherwise they go unused)
    TileChunk ch;
    if (wave == 0) {
        int per, l0, l1;
        walk_range(P, lane, per, l0, l1);
        load_tile_chunk(P.tiles + (int64_t)row * P.geo.ntiles, l0, l1, ch);
    }
    const RowDraw D = P.draws[row];
    if (D.kind == DRAW_RESIDUAL || (P.theta && D.kind == DRAW_BONUS)) {
        if (wave == 0) draw_residual_row<DT, AL>(P, D, row, lane, ch);
    } else if (D.kind == DRAW_BONUS) {
        draw_bonus_row<DT, AL>(P, D, row, lane, wave, s_ts);
    }
}

// The drafter's draw (every row a single position, no drafts): the scan and the draw
// in one workgroup per vector, so the draw's inputs never pass through memory.
template <int DT, bool AL>
__global__ __launch_bounds__(kBlock) void scan_draw_kernel(Params P)
{
    __shared__ ScanLds sh;
    __shared__ double s_ts[kPieceTiles<DT>];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t row = blockIdx.x;
    const RowDraw D = scan_row<DT>(P, row, true, sh);
    if (D.kind == DRAW_BONUS) draw_bonus_row<DT, AL>(P, D, row, lane, wave, s_ts);
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

hipError_t launch_scan(const Params &P, hipStream_t s, int dtype, bool ee)
{
    const void *fn = dtype == 0 ? (ee ? (const void *)scan_kernel<0, true> : (const void *)scan_kernel<0, false>)
                                : (ee ? (const void *)scan_kernel<1, true> : (const void *)scan_kernel<1, false>);
    return launch(fn, (int64_t)P.B, kBlock, P, s);
}

// Workgroups per row of scan_tiles_kernel: enough to give every CU a workgroup, each
// with at least 32 tiles of the row.
int32_t scan_tiles_split(int32_t B, int32_t ntiles)
{
    static int cus = 0;
    if (cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    int64_t S = B > 0 ? ((int64_t)cus + B - 1) / B : 1;
    const int64_t cap = ntiles / 32;
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    return (int32_t)S;
}

// bf16 only: fp32 rows keep the separate scan and verify_kernel_f32, whose residual
// weights come from the hardware exp2 and cost less than the fp64 terms of tile_sums
hipError_t launch_scan_tiles(const Params &P, hipStream_t s, bool aligned, bool ee)
{
    const void *fn = ee ? (aligned ? (const void *)scan_tiles_kernel<0, true, true>
                                   : (const void *)scan_tiles_kernel<0, false, true>)
                        : (aligned ? (const void *)scan_tiles_kernel<0, true, false>
                                   : (const void *)scan_tiles_kernel<0, false, false>);
    return launch(fn, (int64_t)P.B * P.st_split, kScanTileBlock, P, s);
}

hipError_t launch_verify(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)verify_kernel<true> : (const void *)verify_kernel<false>)
        : (aligned ? (const void *)verify_kernel_f32<true> : (const void *)verify_kernel_f32<false>);
    return launch(fn, (int64_t)P.B * P.geo.ndraw, kBlock, P, s);
}

hipError_t launch_ee_init(const Params &P, hipStream_t s)
{
    int64_t blocks = ((int64_t)P.B + kBlock - 1) / kBlock;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    return launch((const void *)ee_init_kernel, blocks, kBlock, P, s);
}

hipError_t launch_ee_step(const Params &P, hipStream_t s, int dtype)
{
    const void *fn = dtype == 0 ? (const void *)ee_step_kernel<0> : (const void *)ee_step_kernel<1>;
    return launch(fn, P.B, kEeWaves * 64, P, s);
}

hipError_t launch_scan_draw(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)scan_draw_kernel<0, true> : (const void *)scan_draw_kernel<0, false>)
        : (aligned ? (const void *)scan_draw_kernel<1, true> : (const void *)scan_draw_kernel<1, false>);
    return launch(fn, P.B, kBlock, P, s);
}

hipError_t launch_draw_final(const Params &P, hipStream_t s, int dtype, bool aligned)
{
    const void *fn = dtype == 0
        ? (aligned ? (const void *)draw_final_kernel<0, true> : (const void *)draw_final_kernel<0, false>)
        : (aligned ? (const void *)draw_final_kernel<1, true> : (const void *)draw_final_kernel<1, false>);
    return launch(fn, P.B, kBlock, P, s);
}

}  // namespace sv
