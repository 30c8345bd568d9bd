// Device code of the accepted-path commit (JetFlow technical summary,
// sections 1 and 4: the target keeps the longest drafted branch it agrees
// with; its tokens join the context, so their K/V rows join the paged cache).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// accepted-path commit: one workgroup per request.  Node j of the request is
// on the accepted node's root path iff bit j of that node's ancestor mask is
// set, and it is the token at position L + depth[j] - 1, so the path needs no
// walk: the workgroup gathers the path's rows by depth, checks every target
// page, then copies the rows 16 bytes per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void commit_kernel(CommitParams p)
{
    __shared__ int32_t src_row[kMaxTree];   // tree row of the path node at depth d + 1
    __shared__ int64_t dst_row[kMaxTree];   // cache row of position L + d
    const int b = blockIdx.x;
    const int j = threadIdx.x;
    typedef const __attribute__((address_space(4))) int32_t *cint_p;
    const int32_t off = ((cint_p)p.tree_off)[b];
    const int32_t end = ((cint_p)p.tree_off)[b + 1];
    const int32_t T = end - off;
    const int32_t L = ((cint_p)p.prefix_len)[b];
    const int32_t a = ((cint_p)p.accepted)[b];
    // request-level checks, identical in every thread (uniform exits)
    int st = kTreeOk;
    if (T < 0 || T > p.max_tree || off < 0 || end > p.N || (b == 0 && off != 0) ||
        (b == p.B - 1 && end != p.N))
        st = kTreeBadOffsets;
    else if (L < 0)
        st = kTreeBadPrefix;
    else if (a < -1 || a >= T)
        st = kCommitBadAccepted;
    if (st != kTreeOk || a == -1) {
        if (j == 0) {
            p.status[b] = st;
            p.new_prefix_len[b] = L;
        }
        return;
    }
    const int32_t da = min(max(p.depth[off + a], 0), T);   // path length
    // the path has one node per depth: as many mask bits as its length
    int pc = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w)
        pc += __builtin_popcountll(p.anc_mask[(int64_t)(off + a) * kMaskWords + w]);
    src_row[j] = -1;
    __syncthreads();
    // gather: the path node at depth d + 1 goes to src_row[d]
    if (j < T) {
        const uint64_t word = p.anc_mask[(int64_t)(off + a) * kMaskWords + (j >> 6)];
        if ((word >> (j & 63)) & 1ull) {
            const int d = p.depth[off + j] - 1;
            if (d >= 0 && d < da)
                src_row[d] = off + j;
        }
    }
    __syncthreads();
    // the plan data must name one node per depth (it does when it comes from a
    // successful plan of this tree); then every target position needs a page
    bool incomplete = (j < da && src_row[j] < 0) || pc != da;
    if (__syncthreads_or(incomplete)) {
        if (j == 0) {
            p.status[b] = kCommitBadPlan;
            p.new_prefix_len[b] = L;
        }
        return;
    }
    bool bad = false;
    if (j < da) {
        const int64_t t = (int64_t)L + j;
        const int64_t pi = t >> p.page_shift;
        int32_t page = -1;
        if (pi < p.max_pages)
            page = p.block_table[(int64_t)b * p.max_pages + pi];
        bad = page < 0 || page >= p.num_pages;
        dst_row[j] = ((int64_t)page << p.page_shift) + (t & ((1 << p.page_shift) - 1));
    }
    if (__syncthreads_or(bad)) {
        if (j == 0) {
            p.status[b] = kCommitBadPage;
            p.new_prefix_len[b] = L;
        }
        return;
    }
    // copy da rows of K and V, 16 bytes per thread per step
    const int cpr = p.row_bytes >> 4;   // 16-byte chunks per row
    const int total = da * cpr;
    for (int c = j; c < total; c += 256) {
        const int d = c / cpr;
        const int o = (c - d * cpr) << 4;
        const int64_t s = (int64_t)src_row[d] * p.row_bytes + o;
        const int64_t t = dst_row[d] * p.row_bytes + o;
        const u32x4 kv = *(const u32x4 *)(p.k_tree + s);
        const u32x4 vv = *(const u32x4 *)(p.v_tree + s);
        *(u32x4 *)(p.k_cache + t) = kv;
        *(u32x4 *)(p.v_cache + t) = vv;
    }
    if (j == 0) {
        p.status[b] = kTreeOk;
        p.new_prefix_len[b] = L + da;
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_commit(const CommitParams &p, hipStream_t stream)
{
    if (p.B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(commit_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
