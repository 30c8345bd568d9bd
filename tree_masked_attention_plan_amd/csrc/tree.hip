// Device code of best-first draft-tree construction (JetFlow technical
// summary, section 2, tree construction: cumulative draft log-probability
// ranks the candidates; best-first expansion to the token budget).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

// ---------------------------------------------------------------------------
// best-first draft trees: one wave per request.
//
// Equal scores go to the earlier push.  In the sequential definition the
// root's children are pushes 0..K-1 and node i's children K + K*i .. +K-1,
// i.e. pushes are ordered by (parent + 1, token): that pair, with the
// candidate's depth appended, is the tie-break tag (cand_tag).
//
// Every child of a node is pushed when the node is popped, and the children
// of one parent leave the pool in the pop order, (score desc, push number
// asc).  So at any time only the best not-yet-popped child of each popped
// node can be the next pop.  The pool holds just that one representative per
// parent: a pop removes the winner w, adds w's next sibling in its parent's
// order (the best sibling whose key is below w's) and w's own best child.
// The pop sequence, and with it every output, is that of the full
// expansion, with at most T + 1 live candidates.  Scores are the same fp32
// sums, in the same order, so every comparison is decided identically.
//
// The pool sits in registers, a few 64-bit keys per lane; a pop is a
// per-lane max and one wave-wide max.
// ---------------------------------------------------------------------------
// A candidate as one 64-bit key whose unsigned order is the pop order:
// larger score first (the float's bits mapped to an order-preserving
// unsigned), then smaller slot.  Key 0 is "no candidate" (also NaN scores,
// which never compare better); -inf is a real score and keys above 0.
__device__ __forceinline__ uint64_t cand_key(float s, int e)
{
    if (e == INT32_MAX || s != s)
        return 0ull;
    if (s == 0.f)
        s = 0.f;   // -0 and +0 are equal scores: one key
    uint32_t u = __builtin_bit_cast(uint32_t, s);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ void cand_of_key(uint64_t k, float &s, int &e)
{
    if (k == 0ull) {
        s = -INFINITY;
        e = INT32_MAX;
        return;
    }
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    s = __builtin_bit_cast(float, u);
    e = (int)(0xFFFFFFFFu - (uint32_t)k);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// max of 64-bit keys inside each row of 16 lanes: every lane of a row gets
// its row's max (DPP rotations)
__device__ __forceinline__ uint64_t row_max_key(uint64_t k)
{
    uint64_t o;
    o = dpp_u64<0x121>(k); k = o > k ? o : k;   // row_ror:1
    o = dpp_u64<0x122>(k); k = o > k ? o : k;   // row_ror:2
    o = dpp_u64<0x124>(k); k = o > k ? o : k;   // row_ror:4
    o = dpp_u64<0x128>(k); k = o > k ? o : k;   // row_ror:8
    return k;
}

// wave-wide max of 64-bit keys; every lane gets the result (the row maxima,
// then the four of them through readlane)
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k)
{
    k = row_max_key(k);
    const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
    const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
    const uint64_t a = r0 > r1 ? r0 : r1, c = r2 > r3 ? r2 : r3;
    return a > c ? a : c;
}

// A candidate's tie-break tag: (parent + 1, k) in the order of the push
// numbers (K + K*parent + k, root children k), which it replaces, with the
// candidate's depth below them (tags are unique without it, so it never
// decides an order): a pop reads parent, token and depth with shifts.
__device__ __forceinline__ int cand_tag(int par, int k, int depth)
{
    return ((par + 1) << 14) | (k << 8) | depth;
}

__global__ __launch_bounds__(64) void build_tree_kernel(TreeParams p)
{
    // pool positions: one per pop plus the root's first child
    constexpr int NS = (kMaxTree + 1 + 63) / 64;
    __shared__ float lps[kTreeMaxLogp];      // this request's log-probabilities
    __shared__ float node_score[kMaxTree];
    // outputs are staged here and written once at the end
    __shared__ int32_t o_parent[kMaxTree], o_choice[kMaxTree];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int K = p.K, T = p.T, Dmax = p.Dmax;
    const float kEmpty = __builtin_nanf("");
    const float *lp = p.logp + (int64_t)b * Dmax * K;
    for (int i = lane; i < Dmax * K; i += 64)
        lps[i] = lp[i];
    for (int i = lane; i < T; i += 64) {
        o_parent[i] = -1;
        o_choice[i] = -1;
        node_score[i] = kEmpty;
    }
    __syncthreads();
    uint64_t slot[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q)
        slot[q] = 0ull;
    // the root's best child opens the pool (key 0: no candidate)
    const uint64_t root_first = wave_max_key(lane < K ? cand_key(lps[lane], cand_tag(-1, lane, 1)) : 0ull);
    if (lane == 0)
        slot[0] = root_first;
    int cnt = 1;   // pool positions used (uniform)
    for (int i = 0; i < T; ++i) {
        uint64_t lb = slot[0];
#pragma unroll
        for (int q = 1; q < NS; ++q)
            lb = slot[q] > lb ? slot[q] : lb;
        const uint64_t kw = wave_max_key(lb);
        if (kw == 0ull)
            break;   // no candidate left: only with NaN inputs (the host checks
                     // that the implicit tree holds T nodes); the remaining
                     // nodes keep parent -1, choice -1, score NaN
        float ws;
        int e;
        cand_of_key(kw, ws, e);                   // uniform
        const int par = (e >> 14) - 1;
        const int k = (e >> 8) & 63;
        const int depth = e & 255;
        const int dp = depth - 1;
        // a node's score was written by lane 0 of this wave in an earlier
        // pop; the wave's LDS accesses complete in program order
        const float sp = par < 0 ? 0.f : node_score[par];
        if (lane == 0) {
            o_parent[i] = par;
            o_choice[i] = k;
            node_score[i] = ws;
        }
        // w's next sibling: the best child of its parent whose key is below
        // w's; and node i's best child, when it is below the depth limit.
        // With K <= 16 the two searches share one pass: sibling candidates
        // in lanes 0..15, child candidates in lanes 16..31.
        uint64_t k_sib, k_child;
        if (K <= 16) {
            // one LDS read for both searches: lanes 0..15 read the parent's
            // row of log-probabilities, lanes 16..31 node i's
            const int j = lane & 15;
            const bool sib = lane < 16;
            const int row = sib ? dp : depth;
            const bool live = lane < 32 && j < K && (sib || depth < Dmax);
            const float v = live ? lps[row * K + j] : 0.f;
            uint64_t key = 0ull;
            if (live) {
                if (sib) {
                    const uint64_t c = cand_key(par < 0 ? v : sp + v, cand_tag(par, j, depth));
                    key = c < kw ? c : 0ull;
                } else {
                    key = cand_key(ws + v, cand_tag(i, j, depth + 1));
                }
            }
            key = row_max_key(key);
            k_sib = readlane_u64(key, 0);
            k_child = readlane_u64(key, 16);
        } else {
            uint64_t ks = 0ull;
            if (lane < K) {
                const float v = lps[dp * K + lane];
                const uint64_t c = cand_key(par < 0 ? v : sp + v, cand_tag(par, lane, depth));
                ks = c < kw ? c : 0ull;
            }
            uint64_t kc = 0ull;
            if (depth < Dmax && lane < K)
                kc = cand_key(ws + lps[depth * K + lane], cand_tag(i, lane, depth + 1));
            k_sib = wave_max_key(ks);
            k_child = wave_max_key(kc);
        }
        // the sibling takes the winner's place; the child takes a new position
#pragma unroll
        for (int q = 0; q < NS; ++q)
            slot[q] = slot[q] == kw ? k_sib : slot[q];
        if (k_child != 0ull) {
            const int pos_lane = cnt & 63, pos_q = cnt >> 6;
#pragma unroll
            for (int q = 0; q < NS; ++q)
                slot[q] = (q == pos_q && lane == pos_lane) ? k_child : slot[q];
            ++cnt;
        }
    }
    __syncthreads();
    for (int i = lane; i < T; i += 64) {
        p.parent[(int64_t)b * T + i] = o_parent[i];
        p.choice[(int64_t)b * T + i] = o_choice[i];
        p.score[(int64_t)b * T + i] = node_score[i];
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_build_tree(const TreeParams &p, hipStream_t stream)
{
    if (p.B == 0 || p.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(build_tree_kernel, dim3(p.B), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
