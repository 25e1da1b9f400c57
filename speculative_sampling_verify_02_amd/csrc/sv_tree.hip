// Greedy verification of candidate trees, after the streaming pass.
//
// A tree of candidate continuations is scored by one forward pass of the target;
// node k's prediction is the first argmax of the target's logits at k, and a node is
// kept when its parent is kept and its token equals the parent's prediction, the
// root (node 0) being the target's own token.  The longest kept path from the root
// is the result (brunomaga.github.io "inference-distillation-speculative-decoding",
// section "Medusa"), the one ending at the lowest node index when several are
// equally long, followed by the prediction at its last node.
//
// tree_kernel runs one workgroup per tree.  The node predictions come from the
// streaming pass's argmax records, merged with LDS atomics on an ordered 64-bit key
// (value, then lowest index).  Whether a node is kept, and its depth, follow from
// pointer jumping over the parent links (log2 of the tree size rounds, every node in
// parallel); the deepest kept node is a block reduction and its path a walk up the
// parents.
#include <limits.h>

#include "sv_internal.h"

namespace sv {

// A float's bits as an unsigned key that sorts like the float (NaN above +inf).
__device__ __forceinline__ uint32_t order_key(float x)
{
    if (x != x) return 0xffffffffu;
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct TreeLds {
    unsigned long long key[kMaxTreeNodes];   // per node: value key << 32 | (INT32_MAX - index)
    int32_t anc[kMaxTreeNodes];
    int32_t par[kMaxTreeNodes];                // tree-local parent (-1 at the root)
    int32_t dep[kMaxTreeNodes];
    int32_t acc[kMaxTreeNodes];
    int32_t tok[kMaxTreeNodes];
    int64_t red[kBlock / 64];
    unsigned long long best;
    int status;
};

__device__ __forceinline__ int64_t block_sum_i64(int64_t v, TreeLds &sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) sh.red[wave] = v;
    __syncthreads();
    int64_t t = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) t += sh.red[w];
    return t;
}

__global__ __launch_bounds__(kBlock) void tree_kernel(TreeParams T)
{
    __shared__ TreeLds sh;
    const int tid = threadIdx.x;
    const int32_t tree = (int32_t)blockIdx.x;

    // offsets: the nodes of earlier trees, and the total
    int64_t before = 0, all = 0;
    for (int32_t j = tid; j < T.B; j += kBlock) {
        const int64_t c = T.counts[j] > 0 ? T.counts[j] : 0;
        all += c;
        if (j < tree) before += c;
    }
    before = block_sum_i64(before, sh);
    all = block_sum_i64(all, sh);
    if (all != T.n_nodes) {
        // counts that do not add up: every tree and every slot is invalid
        for (int64_t s = (int64_t)blockIdx.x * kBlock + tid; s < T.n_nodes; s += (int64_t)gridDim.x * kBlock) {
            T.path[s] = -1;
            T.emitted[s] = -1;
        }
        if (tid == 0) {
            T.n_accepted[tree] = -1;
            if (T.row_status) T.row_status[tree] = ST_BAD_GAMMA;
        }
        return;
    }
    const int64_t off = before;
    const int32_t cnt = T.counts[tree];
    const int n = cnt < 0 ? 0 : (cnt > kMaxTreeNodes ? 0 : cnt);

    // structure and tokens
    if (tid == 0) sh.status = (cnt < 1 || cnt > kMaxTreeNodes) ? ST_BAD_TREE : 0;
    __syncthreads();
    int st = 0;
    for (int k = tid; k < n; k += kBlock) {
        const int32_t par = T.parents[off + k];
        const int32_t tk = T.tokens[off + k];
        if (k == 0 ? par != -1 : (par < 0 || par >= k)) st |= ST_BAD_TREE;
        if (tk < 0 || (int64_t)tk >= T.V) st |= ST_BAD_TOKEN;
        sh.anc[k] = k == 0 ? -1 : par;
        sh.par[k] = k == 0 ? -1 : par;
        sh.tok[k] = tk;
        sh.key[k] = 0ull;
    }
    __syncthreads();
    // predictions: every record of the tree's vectors into its node's key
    // (n <= kMaxTreeNodes nodes of ipv records each: the indices fit 32 bits)
    const uint32_t ipv32 = (uint32_t)T.ipv;
    const uint32_t nrec = (uint32_t)n * ipv32;
    const Partial *rec = T.parts + off * T.ipv;
    for (uint32_t r = tid; r < nrec; r += kBlock) {
        const Partial q = rec[r];
        const uint32_t k = r / ipv32;
        const uint32_t idx = q.idx == INT32_MAX ? 0u : (uint32_t)(INT32_MAX - q.idx);
        atomicMax(&sh.key[k], ((unsigned long long)order_key(q.m) << 32) | idx);
    }
    __syncthreads();
    for (int k = tid; k < n; k += kBlock) {
        const uint32_t hi = (uint32_t)(sh.key[k] >> 32);
        // the maximum must be finite: NaN, +inf, and all -inf (or no record) are not
        if (hi == 0xffffffffu || hi == order_key(INFINITY) || hi <= order_key(-INFINITY)) st |= ST_NONFINITE;
    }
    if (st) atomicOr(&sh.status, st);
    __syncthreads();
    const int status = sh.status;

    if (status == 0) {
        // kept flag and depth per node by pointer jumping: after round t, anc is the
        // ancestor 2^t levels up (-1 past the root), acc whether every node from this
        // one up to (not including) anc has its token equal to its parent's prediction,
        // dep the levels climbed
        for (int k = tid; k < n; k += kBlock) {
            const int32_t par = sh.anc[k];
            const int32_t pred_par = par >= 0 ? INT32_MAX - (int32_t)(uint32_t)(sh.key[par] & 0xffffffffu) : -1;
            sh.acc[k] = par < 0 ? 1 : (sh.tok[k] == pred_par ? 1 : 0);
            sh.dep[k] = par < 0 ? 0 : 1;
        }
        __syncthreads();
        for (int span = 1; span < n; span <<= 1) {
            int32_t na[kMaxTreeNodes / kBlock], nd[kMaxTreeNodes / kBlock], nc[kMaxTreeNodes / kBlock];
#pragma unroll
            for (int s = 0; s < kMaxTreeNodes / kBlock; ++s) {
                const int k = tid + s * kBlock;
                if (k < n) {
                    const int32_t a = sh.anc[k];
                    na[s] = a >= 0 ? sh.anc[a] : -1;
                    nd[s] = sh.dep[k] + (a >= 0 ? sh.dep[a] : 0);
                    nc[s] = sh.acc[k] & (a >= 0 ? sh.acc[a] : 1);
                }
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < kMaxTreeNodes / kBlock; ++s) {
                const int k = tid + s * kBlock;
                if (k < n) {
                    sh.anc[k] = na[s];
                    sh.dep[k] = nd[s];
                    sh.acc[k] = nc[s];
                }
            }
            __syncthreads();
        }
        // the deepest kept node, lowest index on ties
        if (tid == 0) sh.best = 0ull;
        __syncthreads();
        unsigned long long mine = 0ull;
        for (int k = tid; k < n; k += kBlock)
            if (sh.acc[k]) {
                const unsigned long long kk = ((unsigned long long)(uint32_t)sh.dep[k] << 32) |
                                              (uint32_t)(INT32_MAX - k);
                mine = kk > mine ? kk : mine;
            }
        atomicMax(&sh.best, mine);
        __syncthreads();
        const int best = INT32_MAX - (int32_t)(uint32_t)(sh.best & 0xffffffffu);
        const int depth = (int)(sh.best >> 32);
        // the path, root first: one thread walks up the parents (held in LDS) into the
        // anc array (free again), then every slot is written in parallel
        __syncthreads();
        if (tid == 0) {
            int k = best;
            for (int d = depth; d >= 0; --d) {
                sh.anc[d] = k;
                k = sh.par[k];
            }
        }
        __syncthreads();
        for (int d = tid; d < n; d += kBlock) {
            int32_t pnode = -1, e = -1;
            if (d <= depth) pnode = sh.anc[d];
            if (d < depth) e = sh.tok[sh.anc[d + 1]];
            else if (d == depth) e = INT32_MAX - (int32_t)(uint32_t)(sh.key[best] & 0xffffffffu);
            T.path[off + d] = pnode;
            T.emitted[off + d] = e;
        }
        if (tid == 0) {
            T.n_accepted[tree] = depth;
            if (T.row_status) T.row_status[tree] = 0;
        }
    } else {
        for (int64_t d = tid; d < (int64_t)(cnt > 0 ? cnt : 0); d += kBlock) {
            T.path[off + d] = -1;
            T.emitted[off + d] = -1;
        }
        if (tid == 0) {
            T.n_accepted[tree] = -1;
            if (T.row_status) T.row_status[tree] = status;
        }
    }
}

hipError_t launch_tree(const TreeParams &T, hipStream_t s)
{
    if (T.B <= 0) return hipSuccess;
    void *args[] = {const_cast<TreeParams *>(&T)};
    return hipLaunchKernel((const void *)tree_kernel, dim3((unsigned)T.B), dim3(kBlock), args, 0, s);
}

}  // namespace sv
