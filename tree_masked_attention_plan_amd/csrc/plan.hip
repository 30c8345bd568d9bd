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
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_plan(const PlanParams &p, hipStream_t stream)
{
    if (p.B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
