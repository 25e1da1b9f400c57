// The streaming pass of the speculative-sampling verification step for gfx950.
//
// Every logit of every target and draft vector is read exactly once.  The vectors
// are cut into pieces of two halves of 2048 logits; one workgroup per CU owns a
// contiguous range of pieces and its waves take them in order from a counter in LDS,
// each half as four (bf16) or eight (fp32) 16-byte loads per lane with the next
// half's loads in flight while one is reduced.  Per piece a wave writes one record:
// the maximum and the sum of 2^((z - m) c), c = log2(e)/T, over the piece (sampling
// rows) or the first argmax (greedy rows); long bf16 passes collect the records (and
// a filtered call's unit keys) in LDS and write them out after their last piece.  The temperature softmax these summarize is the softened output of
// brunomaga.github.io "inference-distillation-speculative-decoding", section
// "Knowledge distillation", with one T for both models (rayaq.ca "Speculative
// decoding", section "Why the output is exactly the target's").  The wave also keeps
// the logit at each position's draft token when it passes through its registers.
//
// bf16 logits are summed in fp32 (exp2 on the hardware unit, the exponent from one
// fma) and added across lanes in fp64.  fp32 logits are summed term by term in fp64
// (a table-driven exp2): the residual mass of a draft close to the target depends on
// the ratio of the two sums to ~1e-9 relative, below what an fp32 exp can give.
#include <algorithm>

#include "sv_stream.h"

namespace sv {

// Workgroup b owns pieces [b q + min(b, r), (b + 1) q + min(b + 1, r)) of the N
// pieces, q = N / G and r = N % G (from the host: a division here would delay every
// wave's first load by hundreds of scalar instructions).  Its waves take them in order
// from a counter in LDS (each wave's first piece is fixed), so a wave the CU's arbiter
// serves less takes fewer pieces and the workgroup's waves finish together; with one
// workgroup per CU the CUs finish together too.  UM: filtered calls, which also store
// the maximum of every 64 consecutive logits (piece_finish).
// NT: the workgroup's threads (a constant: blockDim would be read from the dispatch
// packet, a memory round trip before the first load).
constexpr int kKeyPieces = 1024;   // 128 KB of staged keys

template <int DT, bool AL, bool UM, int NT, bool ST = false>
__device__ __forceinline__ void stats_body(const Params &P)
{
    __shared__ uint32_t s_next;
    const int lane = threadIdx.x & 63;
    Exp2Tab tab{nullptr, 6};
    if constexpr (DT == 1) {
        __shared__ double s_tab[kTabLen * 64];
        fill_exp2_tab<NT>(s_tab, 64);
        tab.col = s_tab + lane;
    }
    if (threadIdx.x == 0) s_next = 0u;
    __syncthreads();
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const int64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int64_t nwb = NT / 64;
    const int64_t N = P.geo.nitems, G = P.geo.G;   // (the grid)
    int64_t p0, p1;
    if (P.xcd_w[0] > 0) {
        // weighted shares: workgroup b's share is w[b mod 8], its range starts at
        // floor(N W(b) / W(G)) with W(b) the weights of the workgroups before it (the
        // rounding is monotone in W(b) and the last range ends at N, so the ranges
        // still cover every piece once)
        int32_t wsum = 0, pre[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            pre[x] = wsum;
            wsum += P.xcd_w[x];
        }
        auto start = [&](int64_t b) -> int64_t {
            if (b >= G) return N;
            const double w = (double)((b >> 3) * (int64_t)wsum + pre[b & 7]);
            return (int64_t)((double)N * w * P.share_inv);
        };
        p0 = start(blockIdx.x);
        p1 = start((int64_t)blockIdx.x + 1);
    } else {
        const int64_t b = blockIdx.x;
        p0 = b * P.share_q + (b < P.share_r ? b : P.share_r);
        p1 = p0 + P.share_q + (b < P.share_r ? 1 : 0);
    }
    // ST (long bf16 passes): what the pass writes besides its reads is staged in LDS
    // and written out after the workgroup's last piece, in contiguous bursts, instead
    // of piece by piece amid the stream's reads (which made C4's pass 3 % slower for
    // the records, 12 % for the filtered calls' unit keys).  The unit keys of the
    // range's first kKeyPieces pieces (a bit per piece marks those of rows that
    // filter), and the records of its first kRecPieces pieces.
    constexpr bool kStage = DT == 0 && UM && ST;
    uint16_t *keys = nullptr;
    uint32_t *kflag = nullptr;
    if constexpr (kStage) {
        __shared__ uint4 s_keys[kKeyPieces * kPieceUnits / 8];
        __shared__ uint32_t s_kflag[kKeyPieces / 32];
        keys = reinterpret_cast<uint16_t *>(s_keys);
        kflag = s_kflag;
        for (int i = threadIdx.x; i < kKeyPieces / 32; i += NT) s_kflag[i] = 0u;
        __syncthreads();
    }
    constexpr bool kRecStage = DT == 0 && ST;
    constexpr int64_t kRecPieces = kStage ? 1024 : 2048;   // 16 or 32 KB
    Partial *recs = nullptr;
    if constexpr (kRecStage) {
        __shared__ Partial s_rec[kRecPieces];
        recs = s_rec;
    }
    int64_t p = p0 + wave;
    if (p < p1) {
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
    ItemRaw<DT> ra, rb;
    half_begin<DT, AL>(P, v, j, 0, true, ra, lane);
    half_begin<DT, AL>(P, v, j, 1, true, rb, lane);
    // the vector's context by scalar loads (vec_ctx_uniform): as vector loads, reading
    // it would wait for every load in flight, the next piece's included
    VecCtx vc = vec_ctx_uniform(P, v);
    bool filt = UM && row_filters(P, vc.row);   // UM: the row filters (then the maxima only)
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
        piece_half<DT, AL, UM>(P, vc, rm, tc, cj, 0, half_len(P, cj, 0), ra, acc, lane, tab, filt);
        half_begin<DT, AL>(P, v, j, 0, live, ra, lane);
        const int n1 = half_len(P, cj, 1);
        if (n1 > 0) piece_half<DT, AL, UM>(P, vc, rm, tc, cj, 1, n1, rb, acc, lane, tab, filt);
        half_begin<DT, AL>(P, v, j, 1, live, rb, lane);
        const VecCtx vn = vec_ctx_uniform(P, live ? v : 0);
        const bool fn = UM && row_filters(P, vn.row);
        uint16_t *slot = nullptr;
        if (kStage && keys) {
            const int64_t r = cv * ipv + cj - p0;
            if (filt && r < kKeyPieces) {
                slot = keys + r * kPieceUnits;
                if (lane == 0) atomicOr(&kflag[r >> 5], 1u << (r & 31));
            }
        }
        Partial *rslot = nullptr;
        if constexpr (kRecStage) {
            const int64_t r = cv * ipv + cj - p0;
            if (r < kRecPieces) rslot = recs + r;
        }
        piece_finish<DT, UM>(P, vc, rm, tc, cv, cj, acc, filt, slot, rslot);
        if (!live) break;
        vc = vn;
        filt = fn;
        pn = pnn;
    }
    }
    if constexpr (kRecStage) {
        __syncthreads();
        const int64_t n = p1 - p0 < kRecPieces ? p1 - p0 : kRecPieces;
        for (int64_t i = threadIdx.x; i < n; i += NT) P.parts[p0 + i] = recs[i];
    }
    if (kStage && keys) {
        // the staged keys: 8 16-byte words per piece, to [p0, p0 + kKeyPieces) of umax
        __syncthreads();
        const int64_t n = (p1 - p0 < kKeyPieces ? p1 - p0 : kKeyPieces) * (kPieceUnits / 8);
        uint4 *dst = reinterpret_cast<uint4 *>(P.umax + p0 * kPieceUnits);
        const uint4 *src = reinterpret_cast<const uint4 *>(keys);
        for (int64_t i = threadIdx.x; i < n; i += NT) {
            const int64_t r = i / (kPieceUnits / 8);
            if (kflag[r >> 5] & (1u << (r & 31))) dst[i] = src[i];
        }
    }
}

// The early-exit steps' streaming: the pieces of the listed vectors (those of the
// positions each undecided row reads at this step), grid-strided over one-wave
// workgroups, each with its next piece's loads in flight while one is reduced.  Slots
// holding -1 are skipped.  Thread 0 of workgroup 0 also clears the other list
// buffer's counts, which the step kernel after this one fills.
template <int DT, bool AL>
__global__ __launch_bounds__(64) void stats_list_kernel(Params P)
{
    const int lane = threadIdx.x;
    const int buf = P.step & 1;
    Exp2Tab tab{nullptr, 0};
    if constexpr (DT == 1) {   // one shared copy: 64 copies would limit the one-wave workgroups per CU
        __shared__ double s_tab[kTabLen];
        fill_exp2_tab<64>(s_tab, 1);
        __syncthreads();
        tab.col = s_tab;
    }
    if (blockIdx.x == 0 && lane == 0) {
        P.ee_count[2 * (buf ^ 1)] = 0;
        P.ee_count[2 * (buf ^ 1) + 1] = 0;
    }
    if (P.gamma != nullptr && P.hdr->status != 0) return;
    const int64_t ipv = P.geo.ipv;
    const int64_t n = (int64_t)P.ee_count[2 * buf + 1] * ipv;   // pieces listed
    const int64_t G = gridDim.x;
    const int32_t *list = P.ee_vecs[buf];
    int64_t p = blockIdx.x;
    if (p >= n) return;
    auto locate = [&](int64_t q, int64_t &v, int64_t &j) {
        const int64_t s = qdiv(q, ipv, P.geo.inv_ipv);
        j = q - s * ipv;
        v = list[s];
    };
    int64_t v, j;
    locate(p, v, j);
    ItemRaw<DT> ra, rb;
    half_begin<DT, AL>(P, v, j, 0, v >= 0, ra, lane);
    half_begin<DT, AL>(P, v, j, 1, v >= 0, rb, lane);
    VecCtx vc = vec_ctx(P, v >= 0 ? v : 0);
    float cached_T = __builtin_nanf("");
    TempConst tc{};
    for (;;) {
        const int64_t cv = v, cj = j;
        const int64_t pn = p + G;
        const bool live = pn < n;
        if (live) locate(pn, v, j);   // in flight while this piece is reduced
        const bool next = live && v >= 0;
        if (cv >= 0) {
            const int32_t rm = row_mode(P.mode, vc.T);
            if (rm == ROW_SAMPLE && vc.T != cached_T) {
                tc = temp_const<DT>(vc.T);
                cached_T = vc.T;
            }
            PieceAcc<DT> acc;
            piece_half<DT, AL>(P, vc, rm, tc, cj, 0, half_len(P, cj, 0), ra, acc, lane, tab);
            half_begin<DT, AL>(P, v, j, 0, next, ra, lane);
            const int n1 = half_len(P, cj, 1);
            if (n1 > 0) piece_half<DT, AL>(P, vc, rm, tc, cj, 1, n1, rb, acc, lane, tab);
            half_begin<DT, AL>(P, v, j, 1, next, rb, lane);
            const VecCtx vn = vec_ctx(P, next ? v : 0);
            piece_finish<DT>(P, vc, rm, tc, cv, cj, acc);
            vc = vn;
        } else {
            half_begin<DT, AL>(P, v, j, 0, next, ra, lane);
            half_begin<DT, AL>(P, v, j, 1, next, rb, lane);
            vc = vec_ctx(P, next ? v : 0);
        }
        if (!live) break;
        p = pn;
    }
}

// 16-byte aligned rows (the usual case): one workgroup per CU, of 16 waves (bf16) or 12
template <int DT, bool UM, bool ST = false>
__global__ __launch_bounds__(kStatsBlock<DT>) void stats_kernel(Params P)
{
    stats_body<DT, true, UM, kStatsBlock<DT>, ST>(P);
}

// rows that do not start 16-byte aligned: aligned loads, realigned in registers; 12
// waves per CU for bf16, 8 for fp32 (the realignment needs registers of its own)
template <int DT> constexpr int kStatsBlockUnaligned = DT == 0 ? 768 : 512;
template <int DT, bool UM, bool ST = false>
__global__ __launch_bounds__(kStatsBlockUnaligned<DT>) void stats_kernel_unaligned(Params P)
{
    stats_body<DT, false, UM, kStatsBlockUnaligned<DT>, ST>(P);
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

static int stats_block(int dtype, bool aligned)
{
    if (dtype == 0) return aligned ? kStatsBlock<0> : kStatsBlockUnaligned<0>;
    return aligned ? kStatsBlock<1> : kStatsBlockUnaligned<1>;
}

// um: filtered calls; stage: long bf16 passes, which stage their writes in LDS
static const void *stats_fn(int dtype, bool aligned, bool um = false, bool stage = false)
{
    if (stage && dtype == 0) {
        if (um)
            return aligned ? (const void *)stats_kernel<0, true, true>
                           : (const void *)stats_kernel_unaligned<0, true, true>;
        return aligned ? (const void *)stats_kernel<0, false, true> : (const void *)stats_kernel_unaligned<0, false, true>;
    }
    if (um)
        return dtype == 0
            ? (aligned ? (const void *)stats_kernel<0, true> : (const void *)stats_kernel_unaligned<0, true>)
            : (aligned ? (const void *)stats_kernel<1, true> : (const void *)stats_kernel_unaligned<1, true>);
    return dtype == 0
        ? (aligned ? (const void *)stats_kernel<0, false> : (const void *)stats_kernel_unaligned<0, false>)
        : (aligned ? (const void *)stats_kernel<1, false> : (const void *)stats_kernel_unaligned<1, false>);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stats_fn(dtype, aligned), stats_block(dtype, aligned), 0) !=
            hipSuccess || per_cu <= 0)
        per_cu = 1;
    int64_t cap = (int64_t)cus * per_cu;
    if (cap > kMaxStatsGrid) cap = kMaxStatsGrid;
    if (dev < kMaxDev) cache[dev][var] = (int32_t)cap;
    return (int32_t)cap;
}

static const void *stats_list_fn(int dtype, bool aligned)
{
    return dtype == 0
        ? (aligned ? (const void *)stats_list_kernel<0, true> : (const void *)stats_list_kernel<0, false>)
        : (aligned ? (const void *)stats_list_kernel<1, true> : (const void *)stats_list_kernel<1, false>);
}

// One-wave workgroups of the list streaming kernel that fit on the current device at
// once (cached per device and kernel variant).
static int64_t stats_list_grid_cap(int dtype, bool aligned)
{
    constexpr int kMaxDev = 64;
    static int64_t cache[kMaxDev][4] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 4096;
    const int var = dtype * 2 + (aligned ? 1 : 0);
    if (dev < kMaxDev && cache[dev][var] > 0) return cache[dev][var];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stats_list_fn(dtype, aligned), 64, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 8;
    const int64_t cap = (int64_t)cus * per_cu;
    if (dev < kMaxDev) cache[dev][var] = cap;
    return cap;
}

// max_vecs: a bound on the vectors this step lists (the grid covers their pieces, up
// to what fits on the device at once)
hipError_t launch_stats_list(const Params &P, hipStream_t s, int dtype, bool aligned, int64_t max_vecs)
{
    int64_t blocks = max_vecs * P.geo.ipv;
    const int64_t cap = stats_list_grid_cap(dtype, aligned);
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return launch(stats_list_fn(dtype, aligned), blocks, 64, P, s);
}

// Shares of the streaming pass's workgroups by XCD, from clocks of the pass on MI355X
// (device-wide timestamps per workgroup): the workgroups of XCDs 0 and 1 start about
// 0.1-0.3 us after the launch and those of XCDs 2 to 7 about 1.6-2.6 us after it, and
// the odd XCDs stream about 6.5 % slower than the even ones.  With equal shares the
// pass ends with the odd XCDs while the even ones idle (C4: ~197 against ~184 us of
// work).  Each XCD gets work in proportion to its rate times the time it has, T - s,
// for a pass of T = the bytes at 6.4 TB/s.  Only passes of at least 80 us are
// weighted: C4's pass took 1.6 % less time (3.3 us with its records staged), the
// drafter's draw of 2048 vectors (~100 us) 1.3 % less, while shorter ones (13-44 us:
// greedy C3, the drafter's draw of 320 vectors, the tree) took 1-7 % more time over
// the whole step.
// The fp32 pass is bound by arithmetic and keeps equal shares.
static void set_xcd_weights(Params &P, int dtype)
{
    if (dtype != 0 || P.geo.G < 64) return;
    constexpr double kStart[8] = {0.12e-6, 0.25e-6, 1.57e-6, 2.06e-6, 2.5e-6, 2.6e-6, 2.5e-6, 2.5e-6};
    constexpr double kOddRate = 0.935;
    const double T = (double)P.geo.nitems * 2.0 * (double)kItemElems * 2.0 / 6.4e12;
    if (T < 80e-6) return;
    for (int x = 0; x < 8; ++x) {
        const double w = ((x & 1) ? kOddRate : 1.0) * std::max(T - kStart[x], 0.5 * T) / T;
        P.xcd_w[x] = (int32_t)(w * 4096.0 + 0.5);
    }
}

hipError_t launch_stats(const Params &P, hipStream_t s, int dtype, bool aligned, hipEvent_t start, hipEvent_t stop)
{
    Params Q = P;
    set_xcd_weights(Q, dtype);
    // bf16 passes of 60 us or more (at 6.4 TB/s) stage their writes in LDS: C4 202.6 ->
    // 197.1 us, filtered 226.6 -> 202.2 us; on C3 (~35 us) the end-of-pass barrier
    // and burst cost 0.4 us, so shorter passes store piece by piece
    const bool stage = (double)P.geo.nitems * 2.0 * (double)kItemElems * 2.0 / 6.4e12 >= 60e-6;
    const int64_t N = Q.geo.nitems, G = Q.geo.G > 0 ? Q.geo.G : 1;
    Q.share_q = N / G;
    Q.share_r = N % G;
    if (Q.xcd_w[0] > 0) {
        int64_t wsum = 0, pre[8];
        for (int x = 0; x < 8; ++x) {
            pre[x] = wsum;
            wsum += Q.xcd_w[x];
        }
        Q.share_inv = 1.0 / (double)((G >> 3) * wsum + pre[G & 7]);
    }
    return launch_timed(stats_fn(dtype, aligned, P.umax != nullptr, stage), P.geo.G, stats_block(dtype, aligned), Q, s,
                        start, stop);
}

}  // namespace sv
