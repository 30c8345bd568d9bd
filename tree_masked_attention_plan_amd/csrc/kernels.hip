// Device code of the tree-causal paged attention library (gfx950 / CDNA4).
//
// What is computed (JetFlow: Breaking the Scaling Ceiling of Speculative
// Decoding with Parallel Tree Drafting -- technical summary, section 2, core
// architecture, tree-causal attention mask and the branch factorisation): each
// tree node attends to the input prefix and to its own root path inside the
// tree.  The prefix is a paged KV cache addressed through block tables (the
// paged, tree-mask-staged FlashAttention of section 3 is the pages' design for
// Hopper; this file is an independent design for CDNA4).
//
// Kernels:
//   plan_kernel       parent[] -> ancestor bitmask / depth / pos id / status
//   fwd_bf16_kernel   per (request, kv head, row tile, prefix split): packs the
//                     (node x GQA group) query rows into 32-row MFMA tiles,
//                     streams 64-key blocks of the paged prefix through LDS,
//                     then the request's own tree keys under the ancestor
//                     bitmask, with an online softmax in registers
//   merge_kernel      LSE merge of prefix splits (split-K)
//   fwd_f32_kernel    fp32 path: one wave per query row, plain FMA arithmetic
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

static constexpr float kLn2 = 0.69314718055994530942f;
// Rescale the running output only when a row's max grows by more than this
// (in log2 units).  Probabilities then stay below 2^8, far inside fp32 and
// bf16 range, and the rescale (a multiply of the whole accumulator) is rare.
static constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// plan: one workgroup per request, one thread per local node (<= 256)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(PlanParams p)
{
    __shared__ int32_t par[kMaxTree];
    __shared__ int32_t first_bad;
    const int b = blockIdx.x;
    const int j = threadIdx.x;
    const int32_t off = p.tree_off[b];
    const int32_t end = p.tree_off[b + 1];
    const int32_t T = end - off;
    const int32_t L = p.prefix_len[b];
    // request-level checks: identical in every thread, so the early return
    // below is uniform across the workgroup
    const bool bad_off = (T < 0) || (T > p.max_tree) || (off < 0) || (end > p.N) ||
                         (b == 0 && off != 0) || (b == p.B - 1 && end != p.N);
    if (bad_off || L < 0) {
        if (j == 0)
            p.status[b] = bad_off ? kTreeBadOffsets : kTreeBadPrefix;
        return;
    }
    if (j == 0)
        first_bad = INT32_MAX;
    int32_t pj = -1;
    if (j < T) {
        pj = p.parent[off + j];
        par[j] = pj;
    }
    __syncthreads();
    if (j < T && (pj < -1 || pj >= j))
        atomicMin(&first_bad, j);
    __syncthreads();
    const int32_t fb = first_bad;
    if (fb != INT32_MAX) {
        if (j == 0)
            p.status[b] = fb + 1;
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
        uint64_t *row = p.anc_mask + (int64_t)(off + j) * kMaskWords;
        row[0] = w0;
        row[1] = w1;
        row[2] = w2;
        row[3] = w3;
        p.depth[off + j] = d;
        p.pos_id[off + j] = L + d - 1;
    }
    if (j == 0)
        p.status[b] = kTreeOk;
}

// ---------------------------------------------------------------------------
// shared helpers for the forward kernels
// ---------------------------------------------------------------------------
struct Unit {
    int b, c, rt, s;
};

// Workgroups are dealt round-robin to the 8 XCDs (id % 8).  Give each XCD a
// contiguous run of work units so that the row tiles reading the same K/V
// chunk run together on one XCD and share its L2.
__device__ __forceinline__ bool decode_unit(const FwdParams &p, Unit &u)
{
    const int w = blockIdx.x;
    const int id = (w & 7) * p.units_per_xcd + (w >> 3);
    if (id >= p.units)
        return false;
    u.rt = id % p.n_rt;
    int t = id / p.n_rt;
    u.s = t % p.nsplit;
    t /= p.nsplit;
    u.c = t % p.Hkv;
    u.b = t / p.Hkv;
    return true;
}

struct ReqInfo {
    int off, T, L, s_tree, kstart, kend;
};

// Request geometry, clamped so that no input can drive an access outside the
// caller's buffers.
__device__ __forceinline__ ReqInfo request_info(const FwdParams &p, int b, int s)
{
    ReqInfo r;
    int off = p.tree_off[b];
    int end = p.tree_off[b + 1];
    off = min(max(off, 0), p.N);
    end = min(max(end, off), p.N);
    r.off = off;
    r.T = min(end - off, p.max_tree);
    int L = p.prefix_len[b];
    L = min(max(L, 0), p.max_pages << p.page_shift);
    r.L = L;
    r.s_tree = L > 0 ? min(p.nsplit - 1, (L - 1) / p.chunk) : 0;
    r.kstart = s * p.chunk;
    r.kend = (s == r.s_tree) ? L : min(L, r.kstart + p.chunk);
    if (r.kend < r.kstart)
        r.kend = r.kstart;
    return r;
}

// Element offset of the K/V row of prefix token t for kv head c, or -1 when
// the token is outside [0, kend) or its page id is out of range.
__device__ __forceinline__ int64_t prefix_row(const FwdParams &p, const int32_t *bt, int t, int kend, int c)
{
    if (t >= kend)
        return -1;
    const int page = bt[t >> p.page_shift];
    if (page < 0 || page >= p.num_pages)
        return -1;
    const int64_t slot = ((int64_t)page << p.page_shift) + (t & ((1 << p.page_shift) - 1));
    return (slot * p.Hkv + c) * (int64_t)p.D;
}

__device__ __forceinline__ int64_t tree_row(const FwdParams &p, int off, int T, int j, int c)
{
    if (j >= T)
        return -1;
    return ((int64_t)(off + j) * p.Hkv + c) * (int64_t)p.D;
}

// ---------------------------------------------------------------------------
// bf16 forward: D = head dim, NW = waves per workgroup (32 query rows each)
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16): S^T = K Q^T with K as the A
// operand (from LDS) and Q^T as the B operand (registers, loaded once), so a
// lane's 16 accumulators are 16 keys of ONE query row (row = lane % 32; the
// other 16 keys of the 32-key tile are in lane + 32).  Row max / sum then
// need one cross-half exchange per block instead of a 32-lane reduction, and
// the probabilities already sit where the B operand of O^T = V^T P^T wants
// them (same lane, keys along registers).  V is staged in LDS transposed
// (d-major) in the key order those registers imply.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p)
{
    constexpr int NT = NW * 64;
    constexpr int KS = D + 8;    // K row stride in LDS (bf16): +16 B breaks bank aliasing
    constexpr int VS = 64 + 8;   // V^T row stride in LDS (bf16): 144 B per d row
    constexpr int NKC = D / 16;  // 16-wide d chunks (k steps of S^T = K Q^T)
    constexpr int NDT = D / 32;  // 32-wide d tiles of O^T
    constexpr int CH = D / 8;    // 16-byte chunks per K/V row
    constexpr int KP = (64 * CH + NT - 1) / NT;  // K pieces per thread per block
    constexpr int VPC = 16 * CH;                 // V pieces (4 keys x 16 B) per block
    constexpr int VP = (VPC + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

    Unit u;
    if (!decode_unit(p, u))
        return;
    const ReqInfo R = request_info(p, u.b, u.s);
    const int rows = R.T * p.G;
    const int row0 = u.rt * (NW * 32);
    if (row0 >= rows || u.s > R.s_tree)
        return;   // uniform across the workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hh = lane >> 5;   // which half of the wave
    const int lr = lane & 31;   // query row inside the wave's tile
    const int my_row = row0 + wv * 32 + lr;
    const bool row_ok = my_row < rows;
    const int node = row_ok ? my_row / p.G : 0;
    const int qh = u.c * p.G + (row_ok ? my_row - node * p.G : 0);
    const int c = u.c;
    const int32_t *bt = p.block_table + (int64_t)u.b * p.max_pages;
    const uint16_t *kc_base = (const uint16_t *)p.k_cache;
    const uint16_t *vc_base = (const uint16_t *)p.v_cache;
    const uint16_t *kt_base = (const uint16_t *)p.k_tree;
    const uint16_t *vt_base = (const uint16_t *)p.v_tree;

    // Q^T fragments (B operand): lane holds Q[row][kc*16 + hh*8 .. +8]
    bf16x8 qf[NKC];
    {
        const uint16_t *qrow = (const uint16_t *)p.q + ((int64_t)(R.off + node) * p.Hq + qh) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok)
                v = *(const u32x4 *)(qrow + kc * 16 + hh * 8);
            qf[kc] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // tree blocks this workgroup needs (only the split that owns the tree)
    const bool owns_tree = (u.s == R.s_tree);
    uint64_t mw[kMaskWords] = {0, 0, 0, 0};
    int tree_need = 0;
    if (owns_tree) {
        if (row_ok) {
            const uint64_t *mrow = p.anc_mask + (int64_t)(R.off + node) * kMaskWords;
#pragma unroll
            for (int w = 0; w < kMaskWords; ++w)
                mw[w] = (w * 64 < R.T) ? mrow[w] : 0ull;
        }
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w)
            if (__syncthreads_or(mw[w] != 0ull))
                tree_need |= 1 << w;
    }
    const int n_pre = (R.kend - R.kstart + 63) / 64;
    const int n_blocks = n_pre + __builtin_popcount(tree_need);

    // block k -> (is_tree, first key): prefix blocks first, then tree blocks
    auto block_of = [&](int k, bool &is_tree, int &start) {
        if (k < n_pre) {
            is_tree = false;
            start = R.kstart + k * 64;
        } else {
            int r = k - n_pre;
            int m = tree_need;
            for (int i = 0; i < r; ++i)
                m &= m - 1;
            is_tree = true;
            start = (__builtin_ctz(m)) * 64;
        }
    };

    u32x4 kreg[KP];
    u32x4 vreg[VP][4];

    auto load_block = [&](int k) {
        bool is_tree;
        int start;
        block_of(k, is_tree, start);
        const uint16_t *kb = is_tree ? kt_base : kc_base;
        const uint16_t *vb = is_tree ? vt_base : vc_base;
#pragma unroll
        for (int it = 0; it < KP; ++it) {
            const int pc = tid + it * NT;
            const int key = pc / CH;
            const int ch = pc % CH;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (pc < 64 * CH) {
                const int64_t r = is_tree ? tree_row(p, R.off, R.T, start + key, c)
                                          : prefix_row(p, bt, start + key, R.kend, c);
                if (r >= 0)
                    v = *(const u32x4 *)(kb + r + ch * 8);
            }
            kreg[it] = v;
        }
#pragma unroll
        for (int it = 0; it < VP; ++it) {
            const int pc = tid + it * NT;
            const int kq = pc & 15;
            const int dg = pc >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (pc < VPC) {
                    const int key = kq * 4 + i;
                    const int64_t r = is_tree ? tree_row(p, R.off, R.T, start + key, c)
                                              : prefix_row(p, bt, start + key, R.kend, c);
                    if (r >= 0)
                        v = *(const u32x4 *)(vb + r + dg * 8);
                }
                vreg[it][i] = v;
            }
        }
    };

    auto store_block = [&]() {
#pragma unroll
        for (int it = 0; it < KP; ++it) {
            const int pc = tid + it * NT;
            if (pc < 64 * CH) {
                const int key = pc / CH;
                const int ch = pc % CH;
                *(u32x4 *)(Ks + key * KS + ch * 8) = kreg[it];
            }
        }
#pragma unroll
        for (int it = 0; it < VP; ++it) {
            const int pc = tid + it * NT;
            if (pc < VPC) {
                const int kq = pc & 15;
                const int dg = pc >> 4;
                // keys 4kq..4kq+3 land on 4 consecutive positions of the
                // MFMA key order: tile kt, k-chunk a/2, half hq, sub-quad a&1
                const int kt = kq >> 3, qq = kq & 7, a = qq >> 1, hq = qq & 1;
                const int pos = kt * 32 + (a >> 1) * 16 + hq * 8 + (a & 1) * 4;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int wsel = e >> 1;
                    uint32_t x0 = vreg[it][0][wsel], x1 = vreg[it][1][wsel];
                    uint32_t x2 = vreg[it][2][wsel], x3 = vreg[it][3][wsel];
                    uint32_t lo, hi;
                    if (e & 1) {
                        lo = (x0 >> 16) | (x1 & 0xffff0000u);
                        hi = (x2 >> 16) | (x3 & 0xffff0000u);
                    } else {
                        lo = (x0 & 0xffffu) | (x1 << 16);
                        hi = (x2 & 0xffffu) | (x3 << 16);
                    }
                    u32x2 w2 = {lo, hi};
                    *(u32x2 *)(Vt + (dg * 8 + e) * VS + pos) = w2;
                }
            }
        }
    };

    f32x16 acc_o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        acc_o[dt] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max, scaled log2 domain
    float l_run = 0.f;         // this half's partial sum of probabilities
    const float c2 = p.c2;

    if (n_blocks > 0)
        load_block(0);
    for (int k = 0; k < n_blocks; ++k) {
        __syncthreads();   // every wave is done reading the previous block
        store_block();
        __syncthreads();
        if (k + 1 < n_blocks)
            load_block(k + 1);   // global loads in flight during the math below

        bool is_tree;
        int start;
        block_of(k, is_tree, start);

        // which 32-key tiles this wave must compute
        bool active[2];
        uint32_t bits[2] = {0xffffffffu, 0xffffffffu};
        if (is_tree) {
            const int w = start >> 6;
            uint64_t word = 0;
#pragma unroll
            for (int i = 0; i < kMaskWords; ++i)
                word = (i == w) ? mw[i] : word;
            bits[0] = (uint32_t)word;
            bits[1] = (uint32_t)(word >> 32);
            active[0] = __ballot(bits[0] != 0u) != 0ull;
            active[1] = __ballot(bits[1] != 0u) != 0ull;
        } else {
            active[0] = start < R.kend;
            active[1] = start + 32 < R.kend;
        }

        f32x16 s_acc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s_acc[kt] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (active[kt]) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const bf16x8 a = *(const bf16x8 *)(Ks + (kt * 32 + lr) * KS + kc * 16 + hh * 8);
                    s_acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s_acc[kt], 0, 0, 0);
                }
            }
        }

        // masks: lane value i of tile kt is key kt*32 + (i/4)*8 + hh*4 + i%4
        const bool partial = !is_tree && (start + 64 > R.kend);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = (i >> 2) * 8 + hh * 4 + (i & 3);
                bool vis = active[kt];
                if (is_tree)
                    vis = vis && ((bits[kt] >> kk) & 1u);
                else if (partial)
                    vis = vis && (start + kt * 32 + kk < R.kend);
                if (!vis)
                    s_acc[kt][i] = -INFINITY;
            }
        }

        // online softmax
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s_acc[kt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = mx * c2;
        const bool upd = mx2 > m_run + kRescaleSlack;
        if (__ballot(upd) != 0ull) {
            const float m_new = upd ? mx2 : m_run;
            const float alpha = upd ? fast_exp2(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc_o[dt][i] *= alpha;
            m_run = m_new;
        }
        const float mu = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            if (!active[kt])
                continue;
            bf16x8 pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = fast_exp2(__builtin_fmaf(s_acc[kt][i], c2, -mu));
                l_run += pv;
                pb[i >> 3][i & 7] = (__bf16)pv;
            }
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const bf16x8 a = *(const bf16x8 *)(Vt + (dt * 32 + lr) * VS + kt * 32 + kc * 16 + hh * 8);
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], acc_o[dt], 0, 0, 0);
                }
            }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok)
        return;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_run + __builtin_log2f(l_tot) : -INFINITY;
    const int64_t n = R.off + node;
    if (p.nsplit == 1) {
        uint16_t *orow = (uint16_t *)p.out + (n * p.Hq + qh) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const __bf16 e0 = (__bf16)(acc_o[dt][i4 * 4 + 0] * inv);
                const __bf16 e1 = (__bf16)(acc_o[dt][i4 * 4 + 1] * inv);
                const __bf16 e2 = (__bf16)(acc_o[dt][i4 * 4 + 2] * inv);
                const __bf16 e3 = (__bf16)(acc_o[dt][i4 * 4 + 3] * inv);
                u32x2 w2;
                w2[0] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
                w2[1] = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
                *(u32x2 *)(orow + dt * 32 + i4 * 8 + hh * 4) = w2;
            }
        }
        if (hh == 0)
            p.lse[n * p.Hq + qh] = lse2 * kLn2;
    } else {
        float *orow = p.ws_o + (((int64_t)u.s * p.N + n) * p.Hq + qh) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float4 v;
                v.x = acc_o[dt][i4 * 4 + 0] * inv;
                v.y = acc_o[dt][i4 * 4 + 1] * inv;
                v.z = acc_o[dt][i4 * 4 + 2] * inv;
                v.w = acc_o[dt][i4 * 4 + 3] * inv;
                *(float4 *)(orow + dt * 32 + i4 * 8 + hh * 4) = v;
            }
        }
        if (hh == 0)
            p.ws_lse[((int64_t)u.s * p.N + n) * p.Hq + qh] = lse2;
    }
}

// ---------------------------------------------------------------------------
// split-K merge: one wave per (node, q head) row
//   lse = log2 sum_s 2^{lse_s};  O = sum_s 2^{lse_s - lse} O_s
// ---------------------------------------------------------------------------
template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(FwdParams p)
{
    constexpr int PER = D / 64;   // output elements per lane
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const ReqInfo R = request_info(p, b, 0);
    const int node = row / p.Hq;
    const int qh = row - node * p.Hq;
    if (node >= R.T)
        return;
    const int nv = R.s_tree + 1;
    const int64_t n = R.off + node;
    float ls = -INFINITY;
    if (lane < nv)
        ls = p.ws_lse[((int64_t)lane * p.N + n) * p.Hq + qh];
    float mx = ls;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    const float base = (mx == -INFINITY) ? 0.f : mx;
    float wgt = (lane < nv) ? fast_exp2(ls - base) : 0.f;
    float tot = wgt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        tot += __shfl_xor(tot, o);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        acc[e] = 0.f;
    for (int s = 0; s < nv; ++s) {
        const float ws = __shfl(wgt, s);
        const float *src = p.ws_o + (((int64_t)s * p.N + n) * p.Hq + qh) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc[e] += ws * src[e];
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    OutT *dst = (OutT *)p.out + (n * p.Hq + qh) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        dst[e] = (OutT)(acc[e] * inv);
    if (lane == 0)
        p.lse[n * p.Hq + qh] = tot > 0.f ? (base + __builtin_log2f(tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 forward: one wave per (node, q head) row; lanes take keys for the
// scores and head-dim elements for the output.  No split (nsplit == 1).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p)
{
    constexpr int PER = D / 64;
    __shared__ float qs[4][D];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wv;
    const ReqInfo R = request_info(p, b, 0);
    const int node = row / p.Hq;
    const int qh = row - node * p.Hq;
    const bool live = node < R.T;
    const int c = qh / p.G;
    const int64_t n = R.off + (live ? node : 0);
    if (live) {
        const float *q = (const float *)p.q + (n * p.Hq + qh) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            qs[wv][lane + 64 * e] = q[lane + 64 * e];
    }
    __syncthreads();
    if (!live)
        return;   // no barrier after this point
    const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
    const uint64_t *mrow = p.anc_mask + n * kMaskWords;
    const float *kc_base = (const float *)p.k_cache;
    const float *vc_base = (const float *)p.v_cache;
    const float *kt_base = (const float *)p.k_tree;
    const float *vt_base = (const float *)p.v_tree;

    float m_run = -INFINITY, l_run = 0.f;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        acc[e] = 0.f;

    const int n_pre = (R.L + 63) / 64;
    const int n_tree = (R.T + 63) / 64;
    for (int k = 0; k < n_pre + n_tree; ++k) {
        const bool is_tree = k >= n_pre;
        int64_t r;
        if (!is_tree) {
            r = prefix_row(p, bt, k * 64 + lane, R.L, c);
        } else {
            const int j = (k - n_pre) * 64 + lane;
            const uint64_t word = mrow[k - n_pre];
            r = ((word >> lane) & 1ull) ? tree_row(p, R.off, R.T, j, c) : -1;
        }
        const float *kb = is_tree ? kt_base : kc_base;
        const float *vb = is_tree ? vt_base : vc_base;
        float s = -INFINITY;
        if (r >= 0) {
            float d0 = 0.f;
            const float *kr = kb + r;
            for (int d = 0; d < D; ++d)
                d0 = __builtin_fmaf(qs[wv][d], kr[d], d0);
            s = d0 * p.c2;
        }
        float mx = s;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, o));
        const float m_new = fmaxf(m_run, mx);
        if (m_new == -INFINITY)
            continue;   // nothing visible yet in this chunk or before
        const float alpha = fast_exp2(m_run - m_new);
        const float pv = (r >= 0) ? fast_exp2(s - m_new) : 0.f;
        float ps = pv;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            ps += __shfl_xor(ps, o);
        l_run = l_run * alpha + ps;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc[e] *= alpha;
        uint64_t vis = __ballot(r >= 0);
        while (vis) {
            const int jl = __builtin_ctzll(vis);
            vis &= vis - 1;
            const float pj = __shfl(pv, jl);
            const int64_t rj = __shfl(r, jl);
            const float *vr = vb + rj;
#pragma unroll
            for (int e = 0; e < PER; ++e)
                acc[e] = __builtin_fmaf(pj, vr[lane + 64 * e], acc[e]);
        }
        m_run = m_new;
    }
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float *o = (float *)p.out + (n * p.Hq + qh) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        o[lane + 64 * e] = acc[e] * inv;
    if (lane == 0)
        p.lse[n * p.Hq + qh] = l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_plan(const PlanParams &p, hipStream_t stream)
{
    if (p.B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, int NW>
static void launch_fwd_bf16_t(const FwdParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3(p.units_per_xcd * 8), dim3(NW * 64), 0, stream, p);
}

hipError_t launch_fwd(const FwdParams &p, int dtype_fp32, int nw, hipStream_t stream)
{
    if (dtype_fp32) {
        const dim3 row_grid((p.max_tree * p.Hq + 3) / 4, p.B);
        if (p.D == 64)
            hipLaunchKernelGGL((fwd_f32_kernel<64>), row_grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_f32_kernel<128>), row_grid, dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    if (p.D == 64) {
        if (nw == 1) launch_fwd_bf16_t<64, 1>(p, stream);
        else if (nw == 2) launch_fwd_bf16_t<64, 2>(p, stream);
        else launch_fwd_bf16_t<64, 4>(p, stream);
    } else {
        if (nw == 1) launch_fwd_bf16_t<128, 1>(p, stream);
        else if (nw == 2) launch_fwd_bf16_t<128, 2>(p, stream);
        else launch_fwd_bf16_t<128, 4>(p, stream);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const FwdParams &p, hipStream_t stream)
{
    if (p.nsplit == 1)
        return hipSuccess;
    const dim3 row_grid((p.max_tree * p.Hq + 3) / 4, p.B);
    if (p.D == 64)
        hipLaunchKernelGGL((merge_kernel<64, __bf16>), row_grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((merge_kernel<128, __bf16>), row_grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
