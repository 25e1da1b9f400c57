// Internal definitions of the spec_verify HIP library: workspace layout, kernel
// parameters and small device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------------------
// geometry constants
// ---------------------------------------------------------------------------
constexpr int kBlock = 256;              // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kUnitElems = 8;            // logits a lane handles per "unit"
constexpr int kTileUnits = 64;           // pass-2 tile: one unit per lane of a wave
constexpr int kTileElems = kTileUnits * kUnitElems;   // 512 logits
constexpr int kTilesPerSeg = 16;         // pass-2 segment: 16 tiles = 8192 logits
constexpr int kUnroll = 4;               // units per thread per pass-1 iteration
constexpr int kXcds = 8;                 // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int64_t kTargetWorkgroups = 2048;   // pass-1 grid goal (8 per CU)
constexpr int64_t kMinSegUnits = 512;    // pass-1 segment floor (2 units per thread)
constexpr double kLog2e = 1.44269504088896340736;

// row status bits (mirror SV_ROW_* of the public header)
enum : int32_t {
    ST_BAD_TOKEN = 1,
    ST_Q_ZERO = 2,
    ST_NONFINITE = 4,
    ST_BAD_GAMMA = 8,
    ST_ZERO_RESID = 16,
    ST_BAD_TEMP = 32,
    ST_INVALID = ST_BAD_TOKEN | ST_NONFINITE | ST_BAD_GAMMA | ST_BAD_TEMP,
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

struct Partial {           // pass-1 result of one (vector, segment)
    float m;               // sampling: max logit; greedy: max logit
    int32_t idx;           // greedy: first index of the max (INT32_MAX: none)
    double s;              // sampling: sum of 2^((z - m) c); greedy: 0, or NaN if a NaN was seen
};

struct Sum2 {              // pass-2 sums over a tile or a segment
    double w;              // draw weights (residual or bonus)
    double p;              // target probabilities (zero-residual fallback)
};

struct RowDraw {           // what pass 2 needs about one row
    int32_t kind;          // DRAW_NONE / DRAW_RESIDUAL / DRAW_BONUS
    int32_t K;
    int32_t t_row, d_row;  // logit rows of target / draft at position K
    float m_t, m_d;        // maxima at K
    float u;               // the draw's uniform
    int32_t t_slot;        // emitted slot t_off + K
    double S_t, S_d;       // sums of 2^((z - m) c) at K
};

struct Geometry {
    int64_t nunits;        // ceil(V / 8)
    int64_t seg_units;     // pass-1 units per segment
    int32_t nseg;          // pass-1 segments per vector
    int32_t nseg2;         // pass-2 segments per row
    int64_t ntiles;        // pass-2 tiles per vector
};

struct Layout {
    size_t hdr, rows, vec_row, parts, draws, tiles, segs, counters, total;
};

// Pass-1 and pass-2 partitioning; depends only on the shape.
inline Geometry make_geometry(int32_t B, int64_t nT, int64_t V)
{
    Geometry g{};
    g.nunits = (V + kUnitElems - 1) / kUnitElems;
    const int64_t nvec = 2 * nT - B;
    int64_t nseg = nvec > 0 ? (kTargetWorkgroups + nvec - 1) / nvec : 1;
    int64_t max_seg = (g.nunits + kMinSegUnits - 1) / kMinSegUnits;
    if (nseg > max_seg) nseg = max_seg;
    if (nseg < 1) nseg = 1;
    g.seg_units = (g.nunits + nseg - 1) / nseg;
    g.nseg = (int32_t)((g.nunits + g.seg_units - 1) / g.seg_units);
    g.ntiles = (g.nunits + kTileUnits - 1) / kTileUnits;
    g.nseg2 = (int32_t)((g.ntiles + kTilesPerSeg - 1) / kTilesPerSeg);
    return g;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(int32_t B, int64_t nT, int64_t V)
{
    const Geometry g = make_geometry(B, nT, V);
    const int64_t nvec = 2 * nT - B;
    Layout L{};
    size_t off = 0;
    L.hdr = off;      off += align256(sizeof(Header));
    L.rows = off;     off += align256(sizeof(RowInfo) * (size_t)B);
    L.vec_row = off;  off += align256(sizeof(int32_t) * (size_t)nvec);
    L.parts = off;    off += align256(sizeof(Partial) * (size_t)nvec * (size_t)g.nseg);
    L.draws = off;    off += align256(sizeof(RowDraw) * (size_t)B);
    L.tiles = off;    off += align256(sizeof(Sum2) * (size_t)B * (size_t)g.ntiles);
    L.segs = off;     off += align256(sizeof(Sum2) * (size_t)B * (size_t)g.nseg2);
    L.counters = off; off += align256(sizeof(int32_t) * (size_t)B);
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
    int64_t nT, nD, nvec;
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
    int32_t *vec_row;
    Partial *parts;
    RowDraw *draws;
    Sum2 *tiles;
    Sum2 *segs;
    int32_t *counters;
    Geometry geo;
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

// exp((z - m) / T) = 2^((z - m) c) with c = log2(e) / T, split as c_hi + c_lo:
// c_hi is c rounded down to fp32, c_lo >= FLT_MIN > 0 the fp32 remainder, so an
// argument built from them carries c to ~2^-48 and -inf logits stay -inf.
struct TempConst {
    float c_hi, c_lo;
    double c_eff;          // c_hi + c_lo exactly
};

__device__ __forceinline__ TempConst temp_const(float T)
{
    const double c = kLog2e / (double)T;
    TempConst tc;
    tc.c_hi = __double2float_rd(c);
    float lo = (float)(c - (double)tc.c_hi);
    if (!(lo >= 1.175494351e-38f)) lo = 1.175494351e-38f;
    tc.c_lo = lo;
    tc.c_eff = (double)tc.c_hi + (double)tc.c_lo;
    return tc;
}

// Logits whose scaled reference |m c_hi| is below this use the one-rounding
// argument fma(z, c_lo, fma(z, c_hi, -M)); larger ones use (z - m) first.
constexpr float kFastRef = 1073741824.0f;   // 2^30

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load unit `unit` (8 logits) of a vector of V logits; logits past V read as -inf.
// ALIGNED: the vector starts 16-byte aligned and V is a multiple of the vector width.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void load_unit(const void *base, int64_t unit, int64_t V, float *x)
{
    const int64_t e0 = unit * kUnitElems;
    if constexpr (DT == 0) {
        const uint16_t *p = static_cast<const uint16_t *>(base);
        if constexpr (ALIGNED) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[unit];
            x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
            x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
            x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
            x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
        } else {
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e)
                x[e] = (e0 + e < V) ? __uint_as_float((uint32_t)p[e0 + e] << 16) : -INFINITY;
        }
    } else {
        const float *p = static_cast<const float *>(base);
        if constexpr (ALIGNED) {
            const float4 a = reinterpret_cast<const float4 *>(p)[2 * unit];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            if (e0 + 4 < V) {
                const float4 b = reinterpret_cast<const float4 *>(p)[2 * unit + 1];
                x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
            } else {
                x[4] = x[5] = x[6] = x[7] = -INFINITY;
            }
        } else {
#pragma unroll
            for (int e = 0; e < kUnitElems; ++e)
                x[e] = (e0 + e < V) ? p[e0 + e] : -INFINITY;
        }
    }
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

// launchers (sv_kernels.hip)
hipError_t launch_prepare(const Params &P, hipStream_t s);
hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned);
hipError_t launch_scan(const Params &P, hipStream_t s, int dtype);
hipError_t launch_draw(const Params &P, hipStream_t s, int dtype, bool aligned);

}  // namespace sv
