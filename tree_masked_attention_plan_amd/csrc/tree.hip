// Device code of best-first draft-tree construction (JetFlow technical
// summary, section 2, tree construction: cumulative draft log-probability
// ranks the candidates; best-first expansion to the token budget).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

// ---------------------------------------------------------------------------
// best-first draft trees: one wave per request.  Candidate slot e is the e-th
// push (the root's children are 0..K-1, node i's children K + K*i .. +K-1),
// so the slot index is also the tie-break key, and the candidate's parent and
// token follow from it.  Slots are grouped in chunks of 64 whose best
// candidate is kept in LDS (a two-level tournament): a pop is a wave-wide
// argmax over the chunk bests, and afterwards only the chunks that changed
// (the popped slot's, and the one or two the new children land in) are
// re-reduced, one slot per lane.  Scores are the same fp32 sums, in the same
// order, as in the sequential definition, so every comparison is decided
// identically.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool cand_better(float sa, int ea, float sb, int eb)
{
    return sa > sb || (sa == sb && ea < eb);
}

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

// wave-wide best of (s, e) pairs; every lane gets the result.  DPP rotations
// inside each row of 16 lanes (row_ror 1, 2, 4, 8), then the four row maxima
// through readlane: a few cycles per step, no LDS round trips.
__device__ __forceinline__ void wave_best(float &s, int &e)
{
    uint64_t k = cand_key(s, e);
    uint64_t o;
    o = dpp_u64<0x121>(k); k = o > k ? o : k;   // row_ror:1
    o = dpp_u64<0x122>(k); k = o > k ? o : k;   // row_ror:2
    o = dpp_u64<0x124>(k); k = o > k ? o : k;   // row_ror:4
    o = dpp_u64<0x128>(k); k = o > k ? o : k;   // row_ror:8
    const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
    const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
    const uint64_t a = r0 > r1 ? r0 : r1, c = r2 > r3 ? r2 : r3;
    cand_of_key(a > c ? a : c, s, e);
}

__global__ __launch_bounds__(64) void build_tree_kernel(TreeParams p)
{
    constexpr int kChunks = (kTreeMaxPool + 63) / 64;
    // candidate scores; NaN marks a slot that is empty or already popped (NaN
    // never compares better, while -inf is a real score: probability 0)
    __shared__ float pool[kTreeMaxPool];
    __shared__ float cbest_s[kChunks];       // best candidate of each 64-slot chunk
    __shared__ int32_t cbest_e[kChunks];
    __shared__ float lps[kTreeMaxLogp];      // this request's log-probabilities
    __shared__ int32_t node_depth[kMaxTree];
    // outputs are staged here and written once at the end: a global store in
    // the loop would make every pop's barrier wait for a memory round trip
    __shared__ int32_t o_parent[kMaxTree], o_choice[kMaxTree];
    __shared__ float o_score[kMaxTree];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int K = p.K, T = p.T, Dmax = p.Dmax;
    const int cap = K * (T + 1);
    const int nchunks = (cap + 63) / 64;
    const float kEmpty = __builtin_nanf("");
    const float *lp = p.logp + (int64_t)b * Dmax * K;
    for (int i = lane; i < Dmax * K; i += 64)
        lps[i] = lp[i];
    for (int e = lane; e < cap; e += 64)
        pool[e] = kEmpty;
    for (int c = lane; c < nchunks; c += 64) {
        cbest_s[c] = -INFINITY;
        cbest_e[c] = INT32_MAX;
    }
    __syncthreads();
    // re-reduce chunk c from its slots (one per lane)
    auto refresh = [&](int c) {
        const int f = c * 64 + lane;
        float fs = -INFINITY;
        int fe = INT32_MAX;
        if (f < cap) {
            const float v = pool[f];
            if (cand_better(v, f, fs, fe)) {
                fs = v;
                fe = f;
            }
        }
        wave_best(fs, fe);
        if (lane == 0) {
            cbest_s[c] = fs;
            cbest_e[c] = fe;
        }
    };
    // the root's children
    if (lane < K)
        pool[lane] = lps[lane];
    __syncthreads();
    refresh(0);
    if (K > 64)
        refresh(1);
    __syncthreads();
    for (int i = lane; i < T; i += 64) {
        o_parent[i] = -1;
        o_choice[i] = -1;
        o_score[i] = kEmpty;
    }
    __syncthreads();
    for (int i = 0; i < T; ++i) {
        // argmax over the chunk bests
        float ws = -INFINITY;
        int we = INT32_MAX;
        for (int c = lane; c < nchunks; c += 64) {
            const float cs = cbest_s[c];
            const int ce = cbest_e[c];
            if (cand_better(cs, ce, ws, we)) {
                ws = cs;
                we = ce;
            }
        }
        wave_best(ws, we);
        if (we == INT32_MAX)
            break;   // no candidate left: only with NaN inputs (the host checks
                     // that the implicit tree holds T nodes); the remaining
                     // nodes keep parent -1, choice -1, score NaN
        const int e = we;                         // uniform
        const int par = e < K ? -1 : (e - K) / K;
        const int k = e < K ? e : (e - K) % K;
        const int depth = par < 0 ? 1 : node_depth[par] + 1;
        if (lane == 0) {
            o_parent[i] = par;
            o_choice[i] = k;
            o_score[i] = ws;
            node_depth[i] = depth;
            pool[e] = kEmpty;
        }
        // node i pushes its K children (slots K + K*i + c)
        const int e0 = K + K * i;
        const bool push = depth < Dmax;
        if (push && lane < K)
            pool[e0 + lane] = ws + lps[depth * K + lane];
        __syncthreads();
        const int c_pop = e >> 6;
        refresh(c_pop);
        if (push) {
            const int c0 = e0 >> 6, c1 = (e0 + K - 1) >> 6;
            if (c0 != c_pop)
                refresh(c0);
            if (c1 != c0 && c1 != c_pop)
                refresh(c1);
        }
        __syncthreads();   // chunk bests and node_depth before the next pop reads them
    }
    __syncthreads();
    for (int i = lane; i < T; i += 64) {
        p.parent[(int64_t)b * T + i] = o_parent[i];
        p.choice[(int64_t)b * T + i] = o_choice[i];
        p.score[(int64_t)b * T + i] = o_score[i];
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
