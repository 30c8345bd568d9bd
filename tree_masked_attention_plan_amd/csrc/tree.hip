// Device code of best-first draft-tree construction (JetFlow technical
// summary, section 2, tree construction: cumulative draft log-probability
// ranks the candidates; best-first expansion to the token budget).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

// ---------------------------------------------------------------------------
// best-first draft trees, data-parallel: one 256-thread workgroup per request.
//
// The sequential definition pops candidates in the order (score desc, push
// number asc); the root's children are pushes 0..K-1 and node i's children
// K + K*i .. +K-1, so push numbers are ordered by (parent's pop index + 1,
// token).  Node i's pop index is its position in that same order, so the
// order of any two nodes is decided by their scores, then by the positions
// of their parents in the order, then by their tokens -- and positions may
// be taken in any subset that holds both parents: only the relative order of
// nodes matters, and it never changes.
//
// A child never precedes its parent (its score is the parent's plus a
// log-probability <= 0, and on equal scores the parent's push number is the
// smaller), so the T pops are the first T nodes of the whole implicit tree
// in this order, and that set is closed under taking parents.  The kernel
// builds it depth by depth: it keeps the best (at most T) nodes found so far,
// sorted; at depth d it adds the children of the kept depth-d nodes and keeps
// the best T again.  A node that drops out has T better nodes, and so do all
// its descendants, so nothing dropped can come back; after the last depth
// the kept list is exactly the pop sequence, and a node's id is its position
// in it.
//
// Each step places the new children by counting: a child's new position is
// the number of kept nodes above it (a binary search in the sorted list)
// plus the number of new children above it; a kept node moves down by the
// number of new children above it.  Once the list holds T nodes, a child
// below its last node is dropped before counting, so after the first levels
// only a few children per depth are counted.  Scores are the same fp32 sums
// as in the sequential definition (parent score + one log-probability), so
// every comparison is decided identically.
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

// A candidate's tie-break tag: (parent + 1, k) in the order of the push
// numbers (K + K*parent + k, root children k), which it replaces, with the
// candidate's depth below them (tags are unique without it, so it never
// decides an order): a pop reads parent, token and depth with shifts.
__device__ __forceinline__ int cand_tag(int par, int k, int depth)
{
    return ((par + 1) << 14) | (k << 8) | depth;
}

// Inclusive prefix sum of one int per thread over a 256-thread workgroup.
__device__ __forceinline__ int block_scan_incl(int v, int tid, int32_t *wsum)
{
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        v += lane >= o ? t : 0;
    }
    if (lane == 63)
        wsum[wv] = v;
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int w = 0; w < 3; ++w)
        add += w < wv ? wsum[w] : 0;
    __syncthreads();   // wsum is reused by the next scan
    return v + add;
}

// The new position of each of m children (keys ckey) among the n kept nodes
// (keys lkey, sorted best first) and the other children: the kept nodes above
// it (binary search) plus the children above it (all keys are distinct).
// Thread tid ranks children tid, tid + 256, ... (CPT of them, all at once),
// so every child key read from LDS serves all of them, and the reads of a
// block of keys are in flight together.  hist[i] counts the children whose
// binary-search position is i (< n).
template <int CPT>
__device__ __forceinline__ void rank_children(const uint64_t *ckey, int32_t *cpos, int32_t *hist,
                                              const uint64_t *lkey, int n, int m, int tid)
{
    constexpr int NT = 256;
    uint64_t kc[CPT];
    int lo[CPT], hi[CPT], rc[CPT];
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
        const int c = tid + t * NT;
        kc[t] = c < m ? ckey[c] : ~0ull;   // past the children: above every key
        lo[t] = 0;
        hi[t] = n;
        rc[t] = 0;
    }
    // binary searches, interleaved (at most 9 rounds for n <= 256)
    for (int round = 0; round < 9; ++round) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            if (lo[t] < hi[t]) {
                const int mid = (lo[t] + hi[t]) >> 1;
                if (lkey[mid] > kc[t])
                    lo[t] = mid + 1;
                else
                    hi[t] = mid;
            }
        }
    }
    constexpr int U = 8;   // child keys per block of reads
    int c2 = 0;
    for (; c2 + U <= m; c2 += U) {
        uint64_t x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = ckey[c2 + u];
#pragma unroll
        for (int t = 0; t < CPT; ++t)
#pragma unroll
            for (int u = 0; u < U; ++u)
                rc[t] += x[u] > kc[t] ? 1 : 0;
    }
    for (; c2 < m; ++c2) {
        const uint64_t x = ckey[c2];
#pragma unroll
        for (int t = 0; t < CPT; ++t)
            rc[t] += x > kc[t] ? 1 : 0;
    }
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
        const int c = tid + t * NT;
        if (c < m) {
            cpos[c] = lo[t] + rc[t];
            if (lo[t] < n)
                atomicAdd(&hist[lo[t]], 1);
        }
    }
}

// The same positions for many children, E = 2, 4 or 8 per thread (m <=
// 256 E): the children's ranks among themselves come from a bitonic sort of
// their keys, best first, instead of counting all pairs.  Thread tid holds
// positions tid*E .. tid*E+E-1; positions from m on are padding (key 0,
// below every child).  At distance j an exchange stays inside a thread for
// j < E, goes between the lanes of a wave (shuffles) for j < 64 E, and
// through LDS (xk: M keys, xi: M indices; xk may be ckey itself, read
// before the first exchange) beyond.  The sort costs log2(M)(log2(M)+1)/2
// short stages where the count costs m/256 compares of every key per thread.
template <int E>
__device__ __forceinline__ void rank_children_sorted(const uint64_t *ckey, int32_t *cpos, int32_t *hist,
                                                     uint64_t *xk, int32_t *xi, const uint64_t *lkey, int n,
                                                     int m, int tid)
{
    constexpr int M = 256 * E;
    uint64_t k[E];
    int ix[E], lo[E], hi[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int c = tid * E + r;
        k[r] = c < m ? ckey[c] : 0ull;
        ix[r] = c;
        lo[r] = 0;
        hi[r] = c < m ? n : 0;
    }
    // kept nodes above each child: binary searches, interleaved
    for (int round = 0; round < 9; ++round) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
            if (lo[r] < hi[r]) {
                const int mid = (lo[r] + hi[r]) >> 1;
                if (lkey[mid] > k[r])
                    lo[r] = mid + 1;
                else
                    hi[r] = mid;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int c = tid * E + r;
        if (c < m) {
            cpos[c] = lo[r];
            if (lo[r] < n)
                atomicAdd(&hist[lo[r]], 1);
        }
    }
    // children above each child: bitonic sort, descending
    for (int size = 2; size <= M; size <<= 1) {
        for (int j = size >> 1; j > 0; j >>= 1) {   // j and size are uniform
            if (j < E) {
#pragma unroll
                for (int jj = 1; jj < E; jj <<= 1) {
                    if (j != jj)
                        continue;
#pragma unroll
                    for (int r = 0; r < E; ++r) {
                        const int pr = r ^ jj;
                        if (pr <= r)
                            continue;   // each pair once, from its lower position
                        const bool desc = ((tid * E + r) & size) == 0;
                        if (desc ? (k[r] < k[pr]) : (k[r] > k[pr])) {
                            const uint64_t tk = k[r];
                            k[r] = k[pr];
                            k[pr] = tk;
                            const int ti = ix[r];
                            ix[r] = ix[pr];
                            ix[pr] = ti;
                        }
                    }
                }
                continue;
            }
            uint64_t ok[E];
            int oi[E];
            if (j < 64 * E) {
                const int lj = j / E;   // the partner's lane distance, same wave
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const uint32_t h = (uint32_t)__shfl_xor((int)(uint32_t)(k[r] >> 32), lj);
                    const uint32_t l = (uint32_t)__shfl_xor((int)(uint32_t)k[r], lj);
                    ok[r] = ((uint64_t)h << 32) | l;
                    oi[r] = __shfl_xor(ix[r], lj);
                }
            } else {
                __syncthreads();   // the previous readers of xk / xi are done
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    xk[tid * E + r] = k[r];
                    xi[tid * E + r] = ix[r];
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int q = (tid * E + r) ^ j;
                    ok[r] = xk[q];
                    oi[r] = xi[q];
                }
            }
            // the lower position of a pair keeps the better key in a
            // descending run and the worse in an ascending one
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int i = tid * E + r;
                const bool lower = (i & j) == 0;
                const bool desc = (i & size) == 0;
                if ((lower == desc) ? (ok[r] > k[r]) : (ok[r] < k[r])) {
                    k[r] = ok[r];
                    ix[r] = oi[r];
                }
            }
        }
    }
    __syncthreads();   // every child's kept-node count is in cpos
#pragma unroll
    for (int r = 0; r < E; ++r)
        if (ix[r] < m)
            cpos[ix[r]] += tid * E + r;
}

__global__ __launch_bounds__(256) void build_tree_kernel(TreeParams p)
{
    constexpr int NT = 256;
    constexpr int CH = 2048;   // children counted per step
    __shared__ float lps[kTreeMaxLogp];   // this request's log-probabilities
    // the kept nodes, best first, double-buffered: order key, score,
    // parent position (-1: hangs off the prefix), token << 8 | depth
    __shared__ uint64_t lkey[2][kMaxTree];
    __shared__ float lsc[2][kMaxTree];
    __shared__ int32_t lpar[2][kMaxTree];
    __shared__ int32_t lkd[2][kMaxTree];
    // the children of one step
    __shared__ uint64_t ckey[CH];
    __shared__ float csc[CH];
    __shared__ int32_t cinfo[CH];   // (parent position + 1) << 8 | token
    __shared__ int32_t cpos[CH];
    __shared__ int32_t sidx[CH];    // sort scratch: child indices
    // the kept depth-d nodes at the start of depth d: score, and where each
    // is now (-1 once dropped)
    __shared__ float par_sc[kMaxTree];
    __shared__ int32_t par_at[kMaxTree];
    __shared__ int32_t newpos[kMaxTree];
    __shared__ int32_t hist[kMaxTree];
    __shared__ int32_t wsum[4];
    __shared__ int32_t s_count, s_grew;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int K = p.K, T = p.T, Dmax = p.Dmax;
    const float *lp = p.logp + (int64_t)b * Dmax * K;
    for (int i = tid; i < Dmax * K; i += NT)
        lps[i] = lp[i];
    __syncthreads();

    int n = 0;     // kept nodes (uniform)
    int buf = 0;   // which list buffer is current (uniform)
    for (int d = 0; d < Dmax; ++d) {
        // the kept depth-d nodes (for d = 0 the virtual root), compacted
        __syncthreads();   // every thread has read the previous depth's flags
        if (tid == 0) {
            s_count = 0;
            s_grew = 0;
        }
        __syncthreads();
        int nd = 1;
        if (d > 0) {
            for (int i0 = 0; i0 < n; i0 += NT) {
                const int i = i0 + tid;
                const bool at_d = i < n && (lkd[buf][i] & 255) == d;
                const uint64_t bal = __ballot(at_d);
                int wbase = 0;
                if (lane == 0 && bal != 0ull)
                    wbase = atomicAdd(&s_count, __builtin_popcountll(bal));
                wbase = __shfl(wbase, 0);
                if (at_d) {
                    const int idx = wbase + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
                    par_sc[idx] = lsc[buf][i];
                    par_at[idx] = i;
                }
            }
            __syncthreads();
            nd = s_count;
        }
        const int npairs = nd * K;
        for (int base = 0; base < npairs; base += CH) {
            const int cnt = min(CH, npairs - base);
            __syncthreads();
            if (tid == 0)
                s_count = 0;
            __syncthreads();
            const bool full = n == T;
            const uint64_t thr = full ? lkey[buf][T - 1] : 0ull;
            for (int j0 = 0; j0 < cnt; j0 += NT) {
                const int j = j0 + tid;
                bool v = false;
                uint64_t key = 0ull;
                float sc = 0.f;
                int info = 0;
                if (j < cnt) {
                    const int pr = base + j;
                    const int pi = pr / K;            // which parent
                    const int k = pr - pi * K;        // which token
                    const int ppos = d == 0 ? -1 : par_at[pi];
                    if (d == 0 || ppos >= 0) {
                        const float lv = lps[d * K + k];
                        sc = d == 0 ? lv : par_sc[pi] + lv;
                        if (sc == sc) {   // NaN candidates are never chosen
                            key = cand_key(sc, cand_tag(ppos, k, d + 1));
                            v = !full || key > thr;
                            info = ((ppos + 1) << 8) | k;
                        }
                    }
                }
                const uint64_t bal = __ballot(v);
                int wbase = 0;
                if (lane == 0 && bal != 0ull)
                    wbase = atomicAdd(&s_count, __builtin_popcountll(bal));
                wbase = __shfl(wbase, 0);
                if (v) {
                    const int idx = wbase + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
                    ckey[idx] = key;
                    csc[idx] = sc;
                    cinfo[idx] = info;
                }
            }
            if (tid < n)
                hist[tid] = 0;
            __syncthreads();
            const int m = s_count;
            if (m == 0)
                continue;   // uniform
            // new positions: kept nodes above a child (binary search in the
            // sorted list) plus new children above it
            const int cpt = (m + NT - 1) / NT;   // children per thread (uniform)
            // up to 1024 children: count all pairs; more: sort (its 45, 55
            // or 66 dependent stages for 512, 1024 or 2048 positions cost
            // more than the count below that:
            // 32 requests, budget 256, 8 candidates: 72 us counting, 79
            // sorting from 513 children, 87 from 257; 8 requests with 64
            // candidates: 148 -> 130 us sorting from 1025)
            if (cpt == 1)
                rank_children<1>(ckey, cpos, hist, lkey[buf], n, m, tid);
            else if (cpt == 2)
                rank_children<2>(ckey, cpos, hist, lkey[buf], n, m, tid);
            else if (cpt <= 4)
                rank_children<4>(ckey, cpos, hist, lkey[buf], n, m, tid);
            else
                rank_children_sorted<CH / NT>(ckey, cpos, hist, ckey, sidx, lkey[buf], n, m, tid);
            __syncthreads();
            // a kept node at position i moves down by the children above it,
            // those whose binary-search position is <= i
            const int cum = block_scan_incl(tid < n ? hist[tid] : 0, tid, wsum);
            if (tid < n) {
                const int np = tid + cum;
                newpos[tid] = np < T ? np : -1;
            }
            __syncthreads();
            const int nb = buf ^ 1;
            if (tid < n && newpos[tid] >= 0) {
                const int np = newpos[tid];
                const int par = lpar[buf][tid];
                // a kept node's parent precedes it, so it is kept too
                const int par2 = par < 0 ? -1 : newpos[par];
                const int kd = lkd[buf][tid];
                const float sc = lsc[buf][tid];
                lpar[nb][np] = par2;
                lkd[nb][np] = kd;
                lsc[nb][np] = sc;
                lkey[nb][np] = cand_key(sc, cand_tag(par2, kd >> 8, kd & 255));
            }
            for (int c = tid; c < m; c += NT) {
                const int np = cpos[c];
                if (np < T) {
                    const int info = cinfo[c];
                    const int ppos = (info >> 8) - 1;
                    const int k = info & 255;
                    const int par2 = ppos < 0 ? -1 : newpos[ppos];
                    lpar[nb][np] = par2;
                    lkd[nb][np] = (k << 8) | (d + 1);
                    lsc[nb][np] = csc[c];
                    lkey[nb][np] = cand_key(csc[c], cand_tag(par2, k, d + 1));
                    s_grew = 1;
                }
            }
            // where this depth's parents are now
            for (int i = tid; i < nd && d > 0; i += NT) {
                const int q = par_at[i];
                par_at[i] = q < 0 ? -1 : newpos[q];
            }
            n = min(n + m, T);
            buf = nb;
        }
        __syncthreads();
        // no depth d + 1 node was kept: no deeper node can be either
        if (!s_grew)
            break;   // uniform
    }
    // node i is the i-th kept node; positions past the kept nodes are left
    // without a candidate (only when NaN candidates leave fewer than T)
    for (int i = tid; i < T; i += NT) {
        const bool have = i < n;
        const int kd = have ? lkd[buf][i] : 0;
        p.parent[(int64_t)b * T + i] = have ? lpar[buf][i] : -1;
        p.choice[(int64_t)b * T + i] = have ? (kd >> 8) : -1;
        p.score[(int64_t)b * T + i] = have ? lsc[buf][i] : __builtin_nanf("");
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t launch_build_tree(const TreeParams &p, hipStream_t stream)
{
    if (p.B == 0 || p.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(build_tree_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
