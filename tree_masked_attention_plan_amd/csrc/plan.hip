// Device code of the plan: parent array -> ancestor bitmask, depth, position
// id and per-request status (JetFlow technical summary, section 2, core
// architecture: a node sees the prefix and its own root path).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

// ---------------------------------------------------------------------------
// plan: one workgroup per request, one thread per local node (<= 256)
// ---------------------------------------------------------------------------
// The argument block is copied into scalar registers in one go: the empty asm
// makes the copies opaque, so the compiler neither reloads a field where it
// is first used nor chains those loads behind the first global reads.
// Accesses through the copies name the global address space explicitly.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gmem(T *ptr)
{
    return (__attribute__((address_space(1))) T *)ptr;
}

__global__ __launch_bounds__(256) void plan_kernel(PlanParams p_arg)
{
    PlanParams p = p_arg;
    asm volatile("" : "+s"(p.parent), "+s"(p.tree_off), "+s"(p.prefix_len), "+s"(p.anc_mask),
                      "+s"(p.depth), "+s"(p.pos_id), "+s"(p.status), "+s"(p.B), "+s"(p.N),
                      "+s"(p.max_tree));
    __shared__ int32_t par[kMaxTree];
    __shared__ int32_t first_bad;
    const int b = blockIdx.x;
    const int j = threadIdx.x;
    // both request reads in flight before either is waited for
    const int32_t L = gmem(p.prefix_len)[b];
    const int32_t off = gmem(p.tree_off)[b];
    const int32_t end = gmem(p.tree_off)[b + 1];
    __builtin_amdgcn_sched_barrier(0);
    const int32_t T = end - off;
    // request-level checks: identical in every thread, so the early return
    // below is uniform across the workgroup
    const bool bad_off = (T < 0) || (T > p.max_tree) || (off < 0) || (end > p.N) ||
                         (b == 0 && off != 0) || (b == p.B - 1 && end != p.N);
    if (bad_off || L < 0) {
        if (j == 0)
            gmem(p.status)[b] = bad_off ? kTreeBadOffsets : kTreeBadPrefix;
        return;
    }
    if (T <= 64) {
        // A tree of up to 64 nodes fits one wave: lane j holds node j, a
        // ballot finds the first bad parent, and the ancestor sets come by
        // pointer jumping (each round merges the set of the lane's next
        // unmerged ancestor and jumps past it: about log2(depth) rounds of
        // cross-lane reads instead of depth dependent LDS reads).  The other
        // waves have nothing to do.
        if (j >= 64)
            return;   // whole waves
        int32_t jp = j < T ? gmem(p.parent)[off + j] : -1;
        const uint64_t bad = __ballot(j < T && (jp < -1 || jp >= j));
        if (bad != 0ull) {
            if (j == 0)
                gmem(p.status)[b] = (int32_t)__builtin_ctzll(bad) + 1;
            return;
        }
        uint64_t m = j < T ? (1ull << j) : 0ull;
        while (__ballot(jp >= 0) != 0ull) {   // ends: parents precede children
            const int src = jp >= 0 ? jp : j;
            const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)m, src);
            const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(m >> 32), src);
            const int32_t jj = __shfl(jp, src);
            if (jp >= 0) {
                m |= ((uint64_t)hi << 32) | lo;
                jp = jj;
            }
        }
        if (j < T) {
            const int32_t d = __builtin_popcountll(m);
            __attribute__((address_space(1))) uint64_t *row = gmem(p.anc_mask) + (int64_t)(off + j) * kMaskWords;
            row[0] = m;
            row[1] = 0;
            row[2] = 0;
            row[3] = 0;
            gmem(p.depth)[off + j] = d;
            gmem(p.pos_id)[off + j] = L + d - 1;
        }
        if (j == 0)
            gmem(p.status)[b] = kTreeOk;
        return;
    }
    if (j == 0)
        first_bad = INT32_MAX;
    int32_t pj = -1;
    if (j < T) {
        pj = gmem(p.parent)[off + j];
        par[j] = pj;
    }
    __syncthreads();
    if (j < T && (pj < -1 || pj >= j))
        atomicMin(&first_bad, j);
    __syncthreads();
    const int32_t fb = first_bad;
    if (fb != INT32_MAX) {
        if (j == 0)
            gmem(p.status)[b] = fb + 1;
        return;
    }
    if (j < T) {
        // every parent precedes its child, so the walk ends within j+1 steps
        uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
        int32_t d = 0;
        for (int32_t a = j; a >= 0; a = par[a]) {
            const uint64_t bit = 1ull << (a & 63);
            const int word = a >> 6;
            w0 |= word == 0 ? bit : 0;
            w1 |= word == 1 ? bit : 0;
            w2 |= word == 2 ? bit : 0;
            w3 |= word == 3 ? bit : 0;
            ++d;
        }
        __attribute__((address_space(1))) uint64_t *row = gmem(p.anc_mask) + (int64_t)(off + j) * kMaskWords;
        row[0] = w0;
        row[1] = w1;
        row[2] = w2;
        row[3] = w3;
        gmem(p.depth)[off + j] = d;
        gmem(p.pos_id)[off + j] = L + d - 1;
    }
    if (j == 0)
        gmem(p.status)[b] = kTreeOk;
}

// ---------------------------------------------------------------------------
// depth-first relabelling: one workgroup per request, one thread per node.
// The order is the preorder of the forest with roots and children taken in
// increasing local index.  In that order a node comes right after its parent
// and the whole subtrees of its earlier siblings (for a root: the earlier
// roots' subtrees), so with sz = subtree size and
//   es[a] = sum of sz over the earlier siblings of a,
// node v's new index is  sum over a on v's root path of es[a], plus the
// number of v's proper ancestors.  Subtree sizes come from every node adding
// one to each node on its root path (LDS atomics).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void plan_dfs_kernel(PlanDfsParams p_arg)
{
    PlanDfsParams p = p_arg;
    asm volatile("" : "+s"(p.parent), "+s"(p.tree_off), "+s"(p.prefix_len), "+s"(p.perm),
                      "+s"(p.inv_perm), "+s"(p.parent_new), "+s"(p.anc_mask), "+s"(p.depth),
                      "+s"(p.pos_id), "+s"(p.status), "+s"(p.B), "+s"(p.N), "+s"(p.max_tree));
    __shared__ int32_t par[kMaxTree];
    __shared__ int32_t rank[kMaxTree];
    __shared__ int32_t sz[kMaxTree];
    __shared__ int32_t es[kMaxTree];
    __shared__ int32_t bucket[4][kMaxTree + 1];   // per wave: subtree sums by parent + 1
    __shared__ int32_t first_bad;
    const int b = blockIdx.x;
    const int j = threadIdx.x;
    const int32_t L = gmem(p.prefix_len)[b];
    const int32_t off = gmem(p.tree_off)[b];
    const int32_t end = gmem(p.tree_off)[b + 1];
    __builtin_amdgcn_sched_barrier(0);
    const int32_t T = end - off;
    // the plan's checks, in the plan's order (uniform early returns)
    const bool bad_off = (T < 0) || (T > p.max_tree) || (off < 0) || (end > p.N) ||
                         (b == 0 && off != 0) || (b == p.B - 1 && end != p.N);
    if (bad_off || L < 0) {
        if (j == 0)
            gmem(p.status)[b] = bad_off ? kTreeBadOffsets : kTreeBadPrefix;
        return;
    }
    if (j == 0)
        first_bad = INT32_MAX;
    int32_t pj = -1;
    if (j < T) {
        pj = gmem(p.parent)[off + j];
        par[j] = pj;
        sz[j] = 0;
    }
    __syncthreads();
    if (j < T && (pj < -1 || pj >= j))
        atomicMin(&first_bad, j);
    __syncthreads();
    const int32_t fb = first_bad;
    if (fb != INT32_MAX) {
        if (j == 0)
            gmem(p.status)[b] = fb + 1;
        return;
    }
    // subtree sizes: one for every node on each node's root path; the walk
    // ends within j+1 steps since every parent precedes its child
    int32_t d = 0;
    if (j < T) {
        for (int32_t a = j; a >= 0; a = par[a]) {
            atomicAdd(&sz[a], 1);
            ++d;
        }
    }
    __syncthreads();
    // Earlier siblings' subtrees, es[j] = sum of sz[s] over s < j with
    // parent[s] = parent[j]: the siblings in earlier waves through per-wave
    // sums by parent (bucket p + 1, LDS atomics), those in this wave through
    // a scan of its lanes with readlane.
    const int w = j >> 6, l = j & 63;
    for (int q = j; q < 4 * (kMaxTree + 1); q += 256)
        (&bucket[0][0])[q] = 0;
    const int32_t szj = j < T ? sz[j] : 0;
    const int32_t pkey = j < T ? pj : -2;   // never matches a real parent
    __syncthreads();
    if (j < T)
        atomicAdd(&bucket[w][pj + 1], szj);
    int32_t e = 0;
    for (int s = 0; s < 64; ++s) {
        const int32_t ps = __builtin_amdgcn_readlane(pkey, s);
        const int32_t zs = __builtin_amdgcn_readlane(szj, s);
        e += (s < l && ps == pkey) ? zs : 0;
    }
    __syncthreads();
    if (j < T) {
        for (int w2 = 0; w2 < w; ++w2)
            e += bucket[w2][pj + 1];
        es[j] = e;
    }
    __syncthreads();
    if (j < T) {
        int32_t r = d - 1;
        for (int32_t a = j; a >= 0; a = par[a])
            r += es[a];
        // always in [0, T) for a valid tree; kept there regardless, so that
        // no store below can leave the request's rows
        rank[j] = min(max(r, 0), T - 1);
    }
    __syncthreads();
    if (j < T) {
        const int32_t r = rank[j];
        gmem(p.perm)[off + r] = off + j;
        gmem(p.inv_perm)[off + j] = off + r;
        gmem(p.parent_new)[off + r] = pj < 0 ? -1 : rank[pj];
        // the ancestor set in the new labels: bit rank[a] for every a in it
        uint64_t n0 = 0, n1 = 0, n2 = 0, n3 = 0;
        for (int32_t a = j; a >= 0; a = par[a]) {
            const int32_t ra = rank[a];
            const uint64_t bit = 1ull << (ra & 63);
            const int word = ra >> 6;
            n0 |= word == 0 ? bit : 0;
            n1 |= word == 1 ? bit : 0;
            n2 |= word == 2 ? bit : 0;
            n3 |= word == 3 ? bit : 0;
        }
        __attribute__((address_space(1))) uint64_t *row = gmem(p.anc_mask) + (int64_t)(off + r) * kMaskWords;
        row[0] = n0;
        row[1] = n1;
        row[2] = n2;
        row[3] = n3;
        gmem(p.depth)[off + r] = d;
        gmem(p.pos_id)[off + r] = L + d - 1;
    }
    if (j == 0)
        gmem(p.status)[b] = kTreeOk;
}

// ---------------------------------------------------------------------------
// row gather: dst[i] = src[index[i]] for rows of row_bytes bytes (an index
// outside [0, n_src) gives a zero row); V is the copy unit (16 or 4 bytes)
// ---------------------------------------------------------------------------
template <typename V>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherParams p)
{
    const int64_t per_row = p.row_bytes / (int64_t)sizeof(V);
    const V zero = {};
    for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
        const int32_t i = p.index[row];
        const bool ok = i >= 0 && i < p.n_src;
        const V *s = (const V *)p.src + (ok ? (int64_t)i : 0) * per_row;
        V *d = (V *)p.dst + row * per_row;
        for (int64_t e = threadIdx.x; e < per_row; e += blockDim.x)
            d[e] = ok ? s[e] : zero;
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_plan(const PlanParams &p, hipStream_t stream)
{
    if (p.B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_plan_dfs(const PlanDfsParams &p, hipStream_t stream)
{
    if (p.B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_dfs_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherParams &p, hipStream_t stream)
{
    if (p.n_rows == 0)
        return hipSuccess;
    const dim3 grid((unsigned)(p.n_rows < 65536 ? p.n_rows : 65536));
    const bool v16 = p.row_bytes % 16 == 0 && ((uintptr_t)p.src | (uintptr_t)p.dst) % 16 == 0;
    if (v16) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        hipLaunchKernelGGL((gather_rows_kernel<u32x4_t>), grid, dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL((gather_rows_kernel<uint32_t>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace ta
