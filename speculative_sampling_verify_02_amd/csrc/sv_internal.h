// Internal definitions of the spec_verify HIP library: workspace layout, kernel
// parameters and small device helpers shared by the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------------------
// geometry constants
// ---------------------------------------------------------------------------
constexpr int kBlock = 256;              // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kUnitElems = 8;            // logits per draw-tile lane (one 16-byte bf16 load)
constexpr int kTileUnits = 64;           // draw tile: one unit per lane of a wave
constexpr int kTileElems = kTileUnits * kUnitElems;   // 512 logits
constexpr int kTilesPerWave = 2;         // draw: tiles a wave sums with all loads in flight
constexpr int kTilesPerDrawWg = kTilesPerWave * kWaves;   // 8 tiles = 4096 logits
// Streaming pass: a wave reads a half piece of 2048 logits, as loads of 16 bytes per
// lane (lane l's k-th load at byte 1024 k + 16 l): 4 loads (4 KB) for bf16, 8 loads
// (8 KB) for fp32.  (bf16 halves of 4 KB against 8 KB: the pass over 704 vectors of
// 128256 logits took 34.6 against 36.7 us, over 4352 vectors of 152064 200.7 against
// 202.9 us, the finer pieces spreading the end of the pass more evenly; the fp32
// pass, bound by its arithmetic, was slower with 4 KB halves.)
constexpr int64_t kItemElems = 2048;
template <int DT> constexpr int kItemLoads = (int)(kItemElems * (DT == 0 ? 2 : 4) / 1024);
// streaming-pass workgroups, one per CU: bf16 16 waves (4 per SIMD), fp32 12 waves
template <int DT> constexpr int kStatsBlock = DT == 0 ? 1024 : 768;
constexpr int kMaxStatsGrid = 16384;     // cap of the streaming-pass grid
constexpr double kLog2e = 1.44269504088896340736;

// row status bits (mirror SV_ROW_* of the public header)
enum : int32_t {
    ST_BAD_TOKEN = 1,
    ST_Q_ZERO = 2,
    ST_NONFINITE = 4,
    ST_BAD_GAMMA = 8,
    ST_ZERO_RESID = 16,
    ST_BAD_TEMP = 32,
    ST_BAD_TREE = 64,
    ST_INVALID = ST_BAD_TOKEN | ST_NONFINITE | ST_BAD_GAMMA | ST_BAD_TEMP | ST_BAD_TREE,
};

enum : int32_t { ROW_SAMPLE = 0, ROW_GREEDY = 1, ROW_BAD_TEMP = 2 };
enum : int32_t { DRAW_NONE = 0, DRAW_RESIDUAL = 1, DRAW_BONUS = 2 };

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
struct Header {            // call-wide status of a ragged batch
    int32_t status;        // 0 ok, ST_BAD_GAMMA when the gamma array is inconsistent
    int32_t pad[63];
};

struct RowInfo {           // packed offsets of one row (ragged batches)
    int32_t t_off, d_off, gamma, pad;
};

struct Partial {           // streaming-pass result of one piece
    float m;               // max logit (NaN if the overlap holds a NaN; -inf: no finite logit)
    int32_t idx;           // greedy: first index of the max within the vector (INT32_MAX: none)
    double s;              // sampling: sum over the piece of 2^(z c - fl(ref c_hi)) (idx holds ref), or
                           // of 2^((z - m) c) when idx holds a NaN
};

struct VecInfo {           // one streamed vector of a ragged batch (filled by prepare_kernel)
    int32_t row;           // batch row
    int32_t slot;          // index of the position's draft token (d_off + j), -1 at j = gamma
    int32_t x;             // that draft token (when slot >= 0)
    float T;               // the row's temperature
};
static_assert(sizeof(VecInfo) == 16, "vec_ctx_uniform reads a VecInfo as four words");

struct Sum2 {              // draw sums over one tile
    double w;              // draw weights (residual or bonus)
    double p;              // target probabilities (zero-residual fallback)
};

struct RowDraw {           // what the draw needs about one row
    int32_t kind;          // DRAW_NONE / DRAW_RESIDUAL / DRAW_BONUS
    int32_t K;
    int32_t t_row, d_row;  // logit rows of target / draft at position K
    float m_t, m_d;        // maxima at K
    float u;               // the draw's uniform
    int32_t t_slot;        // emitted slot t_off + K
    double S_t, S_d;       // sums of 2^((z - m) c) at K
    float T;
    float theta_t;         // filtering thresholds of target / draft at K (-inf: none)
    float theta_d;
    int32_t pad;
};

// Streaming pass.  The vectors it reads are the target rows (vectors 0 .. nT-1) and,
// in sampling mode, the draft rows (vectors nT .. nT+nD-1).  Each vector is cut into
// ipv pieces of two halves of kItemElems logits (the last piece shorter); piece v ipv + j is
// piece j of vector v, and its record sits at parts[v ipv + j].  Wave w of the grid
// reduces pieces w, w + nwaves, ... .
struct Geometry {
    int64_t nunits;        // ceil(V / 8): draw tiles
    int64_t nvec;          // vectors streamed
    int64_t ie;            // logits per half piece
    int64_t ipv;           // pieces per vector
    int64_t nitems;        // pieces: nvec * ipv
    int32_t G;             // streaming workgroups
    int32_t ntiles;        // draw tiles per vector
    int32_t ndraw;         // draw workgroups per row
    int32_t pad;
    double inv_ipv;        // 1 / ipv, 1 / (gamma + 1), 1 / gamma (dense batches): quotients
    double inv_t, inv_d;   // are estimated in fp64 and corrected by one step
};

struct Layout {
    size_t hdr, rows, vinfo, parts, zx, draws, tiles, total;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t item_elems(int32_t) { return kItemElems; }

inline Geometry make_geometry(int32_t B, int64_t nT, int64_t V, int32_t mode, int32_t dtype,
                              int32_t grid_cap)
{
    Geometry g{};
    const int64_t nD = nT - B;
    g.nunits = ceil_div(V, kUnitElems);
    g.nvec = mode == 1 ? nT : nT + nD;
    g.ie = item_elems(dtype);
    g.ipv = ceil_div(V, 2 * g.ie);
    g.nitems = g.nvec * g.ipv;
    // the workgroups that fit at once, each with an equal share of the pieces
    int64_t G = grid_cap < kMaxStatsGrid ? grid_cap : kMaxStatsGrid;
    if (G > g.nitems) G = g.nitems;
    if (G < 1) G = 1;
    g.G = (int32_t)G;
    g.ntiles = (int32_t)ceil_div(g.nunits, kTileUnits);
    g.ndraw = (int32_t)ceil_div(g.ntiles, kTilesPerDrawWg);
    g.inv_ipv = 1.0 / (double)g.ipv;
    return g;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sized for sampling mode, so it depends only on the shape and dtype.
inline Layout make_layout(int32_t B, int64_t nT, int64_t V, int32_t dtype)
{
    const int64_t nD = nT - B;
    const int64_t nvec = nT + nD;
    const int64_t nitems = nvec * ceil_div(V, 2 * item_elems(dtype));
    const int64_t ntiles = ceil_div(ceil_div(V, kUnitElems), kTileUnits);
    Layout L{};
    size_t off = 0;
    L.hdr = off;      off += align256(sizeof(Header));
    L.rows = off;     off += align256(sizeof(RowInfo) * (size_t)B);
    L.vinfo = off;    off += align256(sizeof(VecInfo) * (size_t)nvec);
    L.parts = off;    off += align256(sizeof(Partial) * (size_t)nitems);
    L.zx = off;       off += align256(sizeof(float) * 2 * (size_t)nD);
    L.draws = off;    off += align256(sizeof(RowDraw) * (size_t)B);
    L.tiles = off;    off += align256(sizeof(Sum2) * (size_t)B * (size_t)ntiles);
    L.total = off;
    return L;
}

// ---------------------------------------------------------------------------
// kernel parameters (passed by value)
// ---------------------------------------------------------------------------
struct Params {
    const void *target;
    const void *draft;
    int64_t V;
    int32_t B;
    int32_t mode;          // SV_SAMPLE / SV_GREEDY
    int64_t nT, nD;
    const int32_t *tokens;
    const float *uniforms;
    const float *temperature;
    const int32_t *gamma;  // NULL: dense with gamma_uniform
    int32_t gamma_uniform;
    int32_t pad0;
    int32_t *n_accepted;
    int32_t *emitted;
    double *p_x, *q_x, *resid;
    int32_t *row_status;
    Header *hdr;
    RowInfo *rows;
    VecInfo *vinfo;        // ragged batches: per-vector row, token and temperature
    Partial *parts;
    float *zx;             // [2 nD]: target then draft logit at each draft token
    RowDraw *draws;
    Sum2 *tiles;
    Geometry geo;
    // early exit (positions read left to right, in chunks): the rows still undecided
    // at the current step and the vectors they read there, double-buffered by step
    // parity
    int32_t *ee_rows[2];      // [B] row ids
    int32_t *ee_vecs[2];      // [max(2 B, nT + nD)] vector ids (-1: none)
    int32_t *ee_count;        // [4]: rows, vectors listed in buffer 0; rows, vectors in buffer 1
    int32_t *ee_status;       // [B] status bits gathered so far
    const int32_t *cache_len; // [B] or null: cache entries before the round
    int32_t *crop_len;        // [B] or null: cache entries to keep after it
    int32_t step;             // chunk being read and decided
    int32_t gamma_max;        // bound on gamma_i given by the caller
    int32_t st_split;         // scan_tiles_kernel: workgroups per row
    int32_t ee_j0, ee_j1;     // this step's positions [ee_j0, ee_j1)
    int32_t ee_j2;            // the next step's end (its positions [ee_j1, ee_j2))
    // streaming pass: relative piece shares of the workgroups on each XCD (workgroup b
    // runs on XCD b mod 8); all zero: equal shares
    int32_t xcd_w[8];
    // streaming pass: N / G and N % G (equal shares), 1 / W(G) (weighted shares)
    int64_t share_q, share_r;
    double share_inv;
    // top-k / top-p filtering of p and q
    const int32_t *top_k;     // [B] or null
    const float *top_p;       // [B] or null
    float *theta;             // [nT + nD] or null: per-vector logit threshold
    // filtered calls: the maximum of every unit of 64 consecutive logits, as a 16-bit
    // key (unit_key), [nT + nD][ipv * 64] (unit u: logits [64 u, 64 u + 64))
    uint16_t *umax;
};

// Units of 64 consecutive logits, 64 to a piece of the streaming pass.
constexpr int kPieceUnits = 64;
inline size_t filter_umax_bytes(int32_t B, int64_t nT, int64_t V)
{
    const int64_t nvec = 2 * nT - B;
    return align256(sizeof(uint16_t) * (size_t)nvec * (size_t)ceil_div(V, 2 * kItemElems) * kPieceUnits);
}

// Early-exit scratch after the verification workspace: two row lists, two vector
// lists (each vector is listed at most once, the first list holds two slots per row),
// the counts and the per-row status.
inline size_t early_exit_list_cap(int32_t B, int64_t nT)
{
    const int64_t all = 2 * nT - B;
    return (size_t)(all > 2 * (int64_t)B ? all : 2 * (int64_t)B);
}
inline size_t early_exit_extra_bytes(int32_t B, int64_t nT)
{
    return align256(sizeof(int32_t) * 2 * (size_t)B) + align256(sizeof(int32_t) * 2 * early_exit_list_cap(B, nT)) +
           align256(sizeof(int32_t) * 4) + align256(sizeof(int32_t) * (size_t)B);
}

// Greedy verification of candidate trees: the streaming pass has left one argmax
// record per piece of every node's vector (nodes packed tree after tree).
constexpr int kMaxTreeNodes = 2048;
struct TreeParams {
    const Partial *parts;
    int64_t ipv;              // records per node vector
    int64_t V;
    int64_t n_nodes;
    int32_t B;                // trees
    int32_t pad;
    const int32_t *counts;    // [B] nodes per tree
    const int32_t *tokens;    // [n_nodes]
    const int32_t *parents;   // [n_nodes], tree-local, -1 for the root
    int32_t *n_accepted;      // [B]
    int32_t *path;            // [n_nodes]
    int32_t *emitted;         // [n_nodes]
    int32_t *row_status;      // [B] or null
};

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
struct RowGeom {
    int64_t t_off, d_off;
    int32_t gamma;
};

__device__ __forceinline__ RowGeom row_geom(const Params &P, int32_t row)
{
    if (P.gamma == nullptr) {
        const int64_t g = P.gamma_uniform;
        return RowGeom{(int64_t)row * (g + 1), (int64_t)row * g, (int32_t)g};
    }
    const RowInfo ri = P.rows[row];
    return RowGeom{ri.t_off, ri.d_off, ri.gamma};
}

// Sampling, greedy, or an unusable temperature for a sampling row.
__device__ __forceinline__ int32_t row_mode(int32_t mode, float T)
{
    if (mode == 1) return ROW_GREEDY;
    if (!(fabsf(T) <= 3.402823466e38f)) return ROW_BAD_TEMP;   // NaN or +-inf
    if (T <= 0.0f) return ROW_GREEDY;
    if (T < 1.175494351e-38f) return ROW_BAD_TEMP;             // subnormal
    return ROW_SAMPLE;
}

// exp((z - m) / T) = 2^((z - m) c) with c = log2(e) / T.
//   bf16 logits (fp32 arithmetic): c_hi = c rounded to fp32 is the scale itself (a
//     relative change of the temperature below 2^-24), c_lo = 0, c_eff = c_hi.
//   fp32 logits: c_eff = c_hi + c_lo carries c to ~2^-48, c_hi rounded down and
//     c_lo >= FLT_MIN the fp32 remainder (the draw's fp32 weights add z c_lo with a
//     second fma; the streaming pass and the other fp64 steps use c_eff).
struct TempConst {
    float c_hi, c_lo;
    double c_eff;
};

template <int DT>
__device__ __forceinline__ TempConst temp_const(float T)
{
    const double c = kLog2e / (double)T;
    TempConst tc;
    if constexpr (DT == 0) {
        tc.c_hi = (float)c;
        tc.c_lo = 0.0f;
        tc.c_eff = (double)tc.c_hi;
    } else {
        tc.c_hi = __double2float_rd(c);
        float lo = (float)(c - (double)tc.c_hi);
        if (!(lo >= 1.175494351e-38f)) lo = 1.175494351e-38f;
        tc.c_lo = lo;
        tc.c_eff = (double)tc.c_hi + (double)tc.c_lo;
    }
    return tc;
}

// fp32 references B = ref * c at or above this magnitude take the (z - m) route:
// the rounding of B (below 2^-4 here) stays a harmless shift of the exponents.
constexpr float kFastRef = 1048576.0f;   // 2^20

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x in fp64: x = n + f with n = rint(x), |f| <= 1/2, and 2^f from its Taylor series
// in f ln 2 to degree 13 (truncation below 5e-18 relative); NaN propagates, very
// negative x (and -inf) give 0.  kExp2Coef holds the series' coefficients (ln 2)^j / j!,
// highest degree first; exp2_f64_by takes them from coef(j), so a kernel can read them
// from constant memory (scalar registers) instead of materializing them.
constexpr double kExp2Coef[14] = {
    0x1.816193166d0f9p-40, 0x1.c3bd650fc2986p-36, 0x1.e8cac7351bb25p-32, 0x1.e4cf5158b8ecap-28,
    0x1.b5253d395e7c4p-24, 0x1.62c0223a5c824p-20, 0x1.ffcbfc588b0c7p-17, 0x1.430912f86c787p-13,
    0x1.5d87fe78a6731p-10, 0x1.3b2ab6fba4e77p-7,  0x1.c6b08d704a0c0p-5,  0x1.ebfbdff82c58fp-3,
    0x1.62e42fefa39efp-1,  1.0};

template <class Coef>
__host__ __device__ __forceinline__ double exp2_f64_by(double x, Coef &&coef)
{
    if (x < -1100.0) x = -1100.0;
    if (x > 1100.0) x = 1100.0;
    const double n = rint(x);
    const double f = x - n;
    double p = coef(0);
#pragma unroll
    for (int j = 1; j < 14; ++j) p = fma(p, f, coef(j));
    return ldexp(p, (int)n);
}

struct Exp2Literal {
    __host__ __device__ double operator()(int j) const { return kExp2Coef[j]; }
};

__host__ __device__ __forceinline__ double exp2_f64(double x) { return exp2_f64_by(x, Exp2Literal{}); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw storage of one unit (8 logits): one 16-byte load for bf16, two for fp32.
template <int DT> struct RawUnit;
template <> struct RawUnit<0> { uint4 a; };
template <> struct RawUnit<1> { float4 a, b; };

// Logits are read once per pass, so every load of them carries the non-temporal
// hint: the lines are not kept in the caches, which measured 10-13 % faster streaming
// than default loads.  kLoadNT is the cache-policy operand of a buffer load (nt).
constexpr int kLoadNT = 2;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 load_nt16f(const void *p)
{
    return __builtin_bit_cast(float4, load_nt16(p));
}

// ALIGNED: the vector starts 16-byte aligned and holds a whole number of 16-byte
// groups; otherwise logits are read one by one (load_tile_unit reads whole tiles of
// such rows with aligned loads).  Logits past V read as -inf.
template <int DT, bool ALIGNED>
__device__ __forceinline__ RawUnit<DT> load_raw(const void *base, int64_t unit, int64_t V)
{
    RawUnit<DT> r;
    const int64_t e0 = unit * kUnitElems;
    if constexpr (DT == 0) {
        const uint16_t *p = static_cast<const uint16_t *>(base);
        if constexpr (ALIGNED) {
            r.a = load_nt16(reinterpret_cast<const uint4 *>(p) + unit);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = (e0 + 2 * k < V) ? (uint32_t)p[e0 + 2 * k] : 0xff80u;
                const uint32_t hi = (e0 + 2 * k + 1 < V) ? (uint32_t)p[e0 + 2 * k + 1] : 0xff80u;
                w[k] = lo | (hi << 16);
            }
            r.a = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        const float *p = static_cast<const float *>(base);
        if constexpr (ALIGNED) {
            r.a = load_nt16f(reinterpret_cast<const float4 *>(p) + 2 * unit);
            if (e0 + 4 < V)
                r.b = load_nt16f(reinterpret_cast<const float4 *>(p) + 2 * unit + 1);
            else
                r.b = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        } else {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (e0 + e < V) ? p[e0 + e] : -INFINITY;
            r.a = make_float4(v[0], v[1], v[2], v[3]);
            r.b = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    return r;
}

// Word 3 of a raw (untyped, offset-addressed) buffer resource on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;

template <int DT>
__device__ __forceinline__ void unpack(const RawUnit<DT> &r, float *x)
{
    if constexpr (DT == 0) {
        x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x);
        x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
        x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z);
        x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
    } else {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
}

// The 16 bytes at byte offset `sb` (0..15) of the 32 bytes lo:hi, dword shift Q.
template <int Q>
__device__ __forceinline__ uint4 funnel16(const uint4 &lo, const uint4 &hi, uint32_t rb)
{
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return make_uint4(__builtin_amdgcn_alignbyte(w[Q + 1], w[Q], rb), __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], rb),
                      __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], rb), __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], rb));
}

__device__ __forceinline__ uint32_t wave_next_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, false);   // lane l <- lane l + 1
}

// Unit tile * 64 + lane of a row that may not start 16-byte aligned (row_base), every
// lane of the wave taking part: aligned 16-byte loads, each clamped to the last aligned
// 16 bytes holding a byte of the array [arr, arr + arr_bytes) (such a block lies in a
// mapped page; what the clamp replaces lies past the row), the bytes moved into place
// with the next lane's block, and logits at V and beyond set to -inf.
__device__ __forceinline__ uint4 funnel16_rt(const uint4 &lo, const uint4 &hi, uint32_t sb)
{
    const uint32_t rb = sb & 3u;
    switch (sb >> 2) {
    case 0: return rb ? funnel16<0>(lo, hi, rb) : lo;
    case 1: return funnel16<1>(lo, hi, rb);
    case 2: return funnel16<2>(lo, hi, rb);
    default: return funnel16<3>(lo, hi, rb);
    }
}

template <int DT>
__device__ __forceinline__ RawUnit<DT> load_tile_unit(const void *row_base, int64_t tile, int64_t V, const void *arr,
                                                      uint64_t arr_bytes, int lane)
{
    constexpr uint64_t ub = DT == 0 ? 16u : 32u;   // bytes per unit
    const uint64_t a = reinterpret_cast<uint64_t>(row_base) + (uint64_t)tile * 64u * ub;
    const uint64_t a0 = a & ~(uint64_t)15;
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(a - a0));
    const uint64_t last = (reinterpret_cast<uint64_t>(arr) + arr_bytes - 1) & ~(uint64_t)15;
    auto blk = [&](uint64_t q) { return load_nt16(reinterpret_cast<const void *>(q < last ? q : last)); };
    RawUnit<DT> r;
    if constexpr (DT == 0) {
        const uint4 b0 = blk(a0 + (uint64_t)lane * 16u);
        const uint4 ext = blk(a0 + 64u * 16u);
        uint4 nx = make_uint4(wave_next_lane(b0.x), wave_next_lane(b0.y), wave_next_lane(b0.z), wave_next_lane(b0.w));
        if (lane == 63) nx = ext;
        r.a = funnel16_rt(b0, nx, sb);
    } else {
        const uint4 b0 = blk(a0 + (uint64_t)lane * 32u), b1 = blk(a0 + (uint64_t)lane * 32u + 16u);
        const uint4 ext = blk(a0 + 64u * 32u);
        uint4 nx = make_uint4(wave_next_lane(b0.x), wave_next_lane(b0.y), wave_next_lane(b0.z), wave_next_lane(b0.w));
        if (lane == 63) nx = ext;
        r.a = __builtin_bit_cast(float4, funnel16_rt(b0, b1, sb));
        r.b = __builtin_bit_cast(float4, funnel16_rt(b1, nx, sb));
    }
    // logits at V and beyond
    const int64_t e0 = (tile * 64 + lane) * kUnitElems;
    if (e0 + kUnitElems > V) {
        if constexpr (DT == 0) {
            uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (e0 + t >= V) w[t / 2] = (t & 1) ? ((w[t / 2] & 0xffffu) | 0xff800000u) : ((w[t / 2] & 0xffff0000u) | 0xff80u);
            r.a = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            float v[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (e0 + t >= V) v[t] = -INFINITY;
            r.a = make_float4(v[0], v[1], v[2], v[3]);
            r.b = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    return r;
}

template <int DT>
__device__ __forceinline__ float load_logit(const void *base, int64_t idx)
{
    if constexpr (DT == 0)
        return __uint_as_float((uint32_t) static_cast<const uint16_t *>(base)[idx] << 16);
    else
        return static_cast<const float *>(base)[idx];
}

__device__ __forceinline__ const void *vec_ptr(const void *base, int dtype, int64_t row, int64_t V)
{
    return static_cast<const char *>(base) + (size_t)row * (size_t)V * (dtype == 0 ? 2u : 4u);
}

// --- wave64 reductions ---
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_min_int(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_or_int(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
    return v;
}
// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ double wave_inclusive_sum(double v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// floor(a / b) for 0 <= a < 2^53 and b >= 1, given inv_b = 1 / b rounded: the fp64
// estimate is off by at most one, which the remainder test corrects.
__device__ __forceinline__ int64_t qdiv(int64_t a, int64_t b, double inv_b)
{
    int64_t q = (int64_t)((double)a * inv_b);
    const int64_t r = a - q * b;
    if (r < 0) --q;
    else if (r >= b) ++q;
    return q;
}

// What the pass needs about one streamed vector.
struct VecCtx {
    int32_t row;
    int32_t slot;   // index of the position's draft token, -1 if none is tested there
    int32_t x;      // that token
    float T;
    bool target;    // a target row (else a draft row)
};

// v: global vector index (target rows first, then draft rows)
// Element i (wave-uniform) of an input that no kernel writes, read as a scalar load
// (through the constant address space).  Scalar loads complete apart from the wave's
// vector loads: waiting for one does not wait for the vector loads in flight.
template <class T>
__device__ __forceinline__ T load_uniform(const T *p, int64_t i)
{
    return ((const __attribute__((address_space(4))) T *)p)[i];
}

// Whether a row of a filtered call has a filter to apply (top-k with 0 < k < V, or
// top-p with 0 < p < 1); row wave-uniform.
__device__ __forceinline__ bool row_filters(const Params &P, int32_t row)
{
    const int64_t k = P.top_k ? load_uniform(P.top_k, row) : 0;
    const float tp = P.top_p ? load_uniform(P.top_p, row) : 1.0f;
    return (k > 0 && k < P.V) || (tp > 0.0f && tp < 1.0f);
}

__device__ __forceinline__ VecCtx vec_ctx(const Params &P, int64_t v)
{
    VecCtx c;
    c.target = v < P.nT;
    if (P.gamma == nullptr) {
        const bool target = c.target;
        const int64_t vloc = target ? v : v - P.nT;
        const int64_t g = P.gamma_uniform;
        const int64_t per = target ? g + 1 : g;   // g > 0 whenever draft vectors exist
        const int64_t row = qdiv(vloc, per, target ? P.geo.inv_t : P.geo.inv_d);
        const int64_t j = vloc - row * per;
        c.row = (int32_t)row;
        c.slot = (P.mode == 0 && j < g) ? (int32_t)(row * g + j) : -1;
        c.x = c.slot >= 0 ? P.tokens[c.slot] : -1;
        c.T = P.mode == 0 ? P.temperature[row] : 0.0f;   // greedy calls may pass no temperatures
    } else {
        const VecInfo vi = P.vinfo[v];
        c.row = vi.row;
        c.slot = P.mode == 0 ? vi.slot : -1;
        c.x = vi.x;
        c.T = vi.T;
    }
    return c;
}

// vec_ctx for a wave-uniform v, with scalar loads (load_uniform): for the streaming
// loops, whose context reads would otherwise wait behind the pieces' loads in flight.
__device__ __forceinline__ VecCtx vec_ctx_uniform(const Params &P, int64_t v)
{
    v = __builtin_amdgcn_readfirstlane((int32_t)v);   // v < nT + nD <= INT32_MAX
    VecCtx c;
    c.target = v < P.nT;
    if (P.gamma == nullptr) {
        const bool target = c.target;
        const int64_t vloc = target ? v : v - P.nT;
        const int64_t g = P.gamma_uniform;
        const int64_t per = target ? g + 1 : g;
        const int64_t row = __builtin_amdgcn_readfirstlane((int32_t)qdiv(vloc, per, target ? P.geo.inv_t : P.geo.inv_d));
        const int64_t j = vloc - row * per;
        c.row = (int32_t)row;
        c.slot = (P.mode == 0 && j < g) ? (int32_t)(row * g + j) : -1;
        c.x = c.slot >= 0 ? load_uniform(P.tokens, c.slot) : -1;
        c.T = P.mode == 0 ? load_uniform(P.temperature, row) : 0.0f;
    } else {
        const int32_t *w = reinterpret_cast<const int32_t *>(P.vinfo + v);   // {row, slot, x, T}
        c.row = load_uniform(w, 0);
        c.slot = P.mode == 0 ? load_uniform(w, 1) : -1;
        c.x = load_uniform(w, 2);
        c.T = __int_as_float(load_uniform(w, 3));
    }
    return c;
}


// --- wave64 all-reductions returning a wave-uniform value: rotations within each
// 16-lane row (DPP row_ror 1, 2, 4, 8) leave every lane with its row's result, and
// the four rows are combined from lanes 0, 16, 32, 48 ---
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const int lo = dpp_i32<CTRL>((int)(uint32_t)b), hi = dpp_i32<CTRL>((int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ float readlane_f32(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// maximum that propagates NaN
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// A unit maximum as a 16-bit key that sorts like it, rounded down: the upper half of
// the float's order-preserving key (exact for bf16 values); 0 for -inf, 0xffff for
// NaN or +inf (finite values take 0x0080 to 0xff7f).
__device__ __forceinline__ uint16_t unit_key(float x)
{
    // selects only: a branch here would split the streaming loop's control flow
    const uint32_t b = __float_as_uint(x);
    uint32_t k = ((b & 0x80000000u) ? ~b : (b | 0x80000000u)) >> 16;
    k = x == -INFINITY ? 0u : k;
    k = x < INFINITY ? k : 0xffffu;
    return (uint16_t)k;
}

__device__ __forceinline__ float wave_umax_f32(float v)
{
    v = nmax(v, dpp_f32<0x121>(v));
    v = nmax(v, dpp_f32<0x122>(v));
    v = nmax(v, dpp_f32<0x124>(v));
    v = nmax(v, dpp_f32<0x128>(v));
    return nmax(nmax(readlane_f32(v, 0), readlane_f32(v, 16)), nmax(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ int wave_umin_i32(int v)
{
    v = min(v, dpp_i32<0x121>(v));
    v = min(v, dpp_i32<0x122>(v));
    v = min(v, dpp_i32<0x124>(v));
    v = min(v, dpp_i32<0x128>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ double wave_usum_f64(double v)
{
    v += dpp_f64<0x121>(v);
    v += dpp_f64<0x122>(v);
    v += dpp_f64<0x124>(v);
    v += dpp_f64<0x128>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// launchers (sv_kernels.hip)
int32_t stats_grid_cap(int dtype, bool aligned);
// A launch of one kernel with its Params.  With events, they are attached to the
// dispatch itself (hipExtLaunchKernel), so they mark the kernel's own start and end
// rather than two extra records on the stream around it; with nothing to launch they
// still mark the (empty) interval.
inline hipError_t launch_timed(const void *fn, int64_t blocks, int threads, const Params &P, hipStream_t s,
                               hipEvent_t start, hipEvent_t stop)
{
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if (blocks <= 0) {
        hipError_t e = hipSuccess;
        if (start) e = hipEventRecord(start, s);
        if (e == hipSuccess && stop) e = hipEventRecord(stop, s);
        return e;
    }
    void *args[] = {const_cast<Params *>(&P)};
    if (!start && !stop) return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), args, 0, s);
    return hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), args, 0, s, start, stop, 0);
}

hipError_t launch_prepare(const Params &P, hipStream_t s);
hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned, hipEvent_t start = nullptr,
                        hipEvent_t stop = nullptr);
hipError_t launch_scan(const Params &P, hipStream_t s, int dtype, bool ee = false);
hipError_t launch_verify(const Params &P, hipStream_t s, int dtype, bool aligned);
int32_t scan_tiles_split(int32_t B, int32_t ntiles);
hipError_t launch_scan_tiles(const Params &P, hipStream_t s, bool aligned, bool ee = false);
hipError_t launch_draw_final(const Params &P, hipStream_t s, int dtype, bool aligned);
hipError_t launch_scan_draw(const Params &P, hipStream_t s, int dtype, bool aligned);
hipError_t launch_tree(const TreeParams &T, hipStream_t s);
hipError_t launch_stats_list(const Params &P, hipStream_t s, int dtype, bool aligned, int64_t max_vecs);
hipError_t launch_ee_init(const Params &P, hipStream_t s);
hipError_t launch_ee_step(const Params &P, hipStream_t s, int dtype);
hipError_t launch_filter(const Params &P, hipStream_t s, int dtype, bool aligned);
int filter_units_num(int64_t V);
hipError_t launch_filter_units(const Params &P, hipStream_t s, int dtype, bool aligned);

}  // namespace sv
