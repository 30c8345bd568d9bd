// Device code of tree-causal paged attention (gfx950 / CDNA4).
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
//   fwd_bf16_kernel   per (request, kv head, row tile, split slot): packs the
//                     (node x GQA group) query rows into 32-row MFMA tiles,
//                     streams 64-key blocks of the paged prefix through LDS,
//                     then the request's own tree keys under the ancestor
//                     bitmask, with an online softmax in registers
//   merge_kernel      LSE merge of the split slots (split-K), one wave per row;
//   merge_lanes_kernel the same for many rows and few splits, lanes per row
//   fwd_f32_kernel    fp32 path: one wave per query row, plain FMA arithmetic
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));   // split partial outputs
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Stores of split partials (rows and (lse, exponent) pairs) with the
// agent-scope bit set: the lines are written through the XCD's L2 instead of
// staying dirty there.  The kernel's end then has no partials to write back
// from the L2s, and the merge kernel, whose rows sit on other XCDs anyway,
// reads them from memory as before.  Same bits; one request of budget 16:
// step 12.22 -> 11.96 us; budget 256: 26.58 -> 25.11 us; 8 requests of
// budget 64: 45.8 -> 44.4 us.  The merge's and the unsplit outputs keep plain
// stores: written through, the merge step slowed 0.4 us and 32 requests of
// budget 256 went 563 -> 586 us; the non-temporal hint instead slowed the
// merge (its reads of such partials) and that batch (641 us).
// Nothing in the kernels loads from global memory after these stores, so
// that the compiler's wait counts, which do not see them, stay exact; a
// 16-byte store needs one wait state before its data registers are written
// again, which the trailing s_nop gives (the hazard check does not look
// inside asm).
template <class P>
__device__ __forceinline__ void store_through(P ptr, u32x4 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 0"
                 :
                 : "v"((uint64_t)(uintptr_t)ptr), "v"(v)
                 : "memory");
}
template <class P>
__device__ __forceinline__ void store_through(P ptr, u32x2 v)
{
    asm volatile("global_store_dwordx2 %0, %1, off sc1"
                 :
                 : "v"((uint64_t)(uintptr_t)ptr), "v"(v)
                 : "memory");
}

static constexpr float kLn2 = 0.69314718055994530942f;
// Rescale the running output only when a row's max grows by more than this
// (in log2 units).  Probabilities then stay below 2^8, far inside fp32 and
// bf16 range, and the rescale (a multiply of the whole accumulator) is rare.
static constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt left at their max)
#define TA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// ---------------------------------------------------------------------------
// shared helpers for the forward kernels
// ---------------------------------------------------------------------------
struct Unit {
    int b, c, rt, s;
};

// The argument copies below are opaque to the compiler, which then no longer
// knows that their pointers address global memory; accesses through them
// name the global address space explicitly (global_ rather than flat_
// instructions, which would also count against lgkmcnt).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gmem(T *ptr)
{
    return (__attribute__((address_space(1))) T *)ptr;
}

// Every kernel argument into scalar registers at once.  Left to itself the
// compiler loads each field of the argument block where it is first used (or
// loads it again later instead of keeping it), and each such load is one
// more dependent scalar-cache round trip.  The empty asm statements make the
// copies opaque values, so they are loaded together here and kept.
__device__ __forceinline__ FwdParams load_args(const FwdParams &in)
{
    FwdParams a = in;
    asm volatile("" : "+s"(a.q), "+s"(a.k_tree), "+s"(a.v_tree), "+s"(a.k_cache), "+s"(a.v_cache),
                      "+s"(a.block_table), "+s"(a.prefix_len), "+s"(a.tree_off), "+s"(a.anc_mask),
                      "+s"(a.out), "+s"(a.lse), "+s"(a.ws_o), "+s"(a.ws_ml));
    asm volatile("" : "+s"(a.B), "+s"(a.N), "+s"(a.Hq), "+s"(a.Hkv), "+s"(a.G), "+s"(a.D),
                      "+s"(a.num_pages), "+s"(a.max_pages), "+s"(a.page_shift), "+s"(a.max_tree),
                      "+s"(a.nsplit), "+s"(a.chunk), "+s"(a.tree_slot), "+s"(a.n_rt), "+s"(a.units),
                      "+s"(a.units_per_xcd), "+s"(a.c2));
    return a;
}

// Workgroups are dealt round-robin to the 8 XCDs (id % 8).  Give each XCD a
// contiguous run of work units so that the row tiles reading the same K/V
// chunk (consecutive ids) run together on one XCD and share its L2.  Units
// are numbered kv head major, then request, so that each XCD's run holds a
// slice of every request: with requests of different prefix lengths no XCD
// gets all of the longest one.
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
    u.b = t % p.B;
    u.c = t / p.B;
    return true;
}

struct ReqInfo {
    int off, T, L, kstart, kend;
    bool owns_tree;   // this unit runs the request's tree phase
};

// Request geometry, clamped so that no input can drive an access outside the
// caller's buffers.  With one split the unit covers the whole prefix and the
// tree.  With nsplit > 1, slot s covers prefix keys [s * chunk, (s + 1) *
// chunk) (a slot past the request's prefix is empty), and the tree phase goes
// either to a slot of its own, the last (tree_slot: the tree runs beside the
// prefix chunks), or to the request's last non-empty chunk (slot 0 for an
// empty prefix).
__device__ __forceinline__ ReqInfo request_info(const FwdParams &p, int b, int s)
{
    // read-only for the whole launch: scalar loads through the constant space
    typedef const __attribute__((address_space(4))) int32_t *cint_p;
    ReqInfo r;
    int off = ((cint_p)p.tree_off)[b];
    int end = ((cint_p)p.tree_off)[b + 1];
    off = min(max(off, 0), p.N);
    end = min(max(end, off), p.N);
    r.off = off;
    r.T = min(end - off, p.max_tree);
    int L = ((cint_p)p.prefix_len)[b];
    L = min(max(L, 0), p.max_pages << p.page_shift);
    r.L = L;
    if (p.nsplit == 1) {
        r.kstart = 0;
        r.kend = L;
        r.owns_tree = true;
    } else if (p.tree_slot && s == p.nsplit - 1) {
        r.kstart = 0;
        r.kend = 0;
        r.owns_tree = true;
    } else {
        r.kstart = s * p.chunk;
        r.kend = max(r.kstart, min(L, r.kstart + p.chunk));
        r.owns_tree = !p.tree_slot && s == (L > 0 ? (L - 1) / p.chunk : 0);
    }
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
// Cross-lane reductions on the VALU (DPP and the gfx950 lane swaps) rather
// than through LDS.  Each step combines a lane with its partner under an
// xor pattern (1, 2 in a quad; the mirrored lane in a half row and in a row;
// the lane 16 and 32 away), so every lane ends with the same value, bit for
// bit: each step adds the same two operands in every lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_f(float v, int ctrl_id)
{
    switch (ctrl_id) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    }
}

// v[l] op v[l ^ 16] and v[l] op v[l ^ 32] in every lane, with the operands in
// the same order in both lanes of a pair (lower row / half first)
template <typename Op>
__device__ __forceinline__ float xor16(float v, Op op)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
template <typename Op>
__device__ __forceinline__ float xor32(float v, Op op)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        v = op(v, dpp_f(v, k));
    return xor32(xor16(v, op), op);
}

// ---------------------------------------------------------------------------
// split-K merge of RB (node, q head) rows by one wave, row ids r0[r] = n * Hq
// + h (rows with on[r] false are skipped):
//   lse = log2 sum_s 2^{lse_s};  O = sum_s 2^{lse_s - lse} O_s
// where O_s = 2^{e_s} P_s and P_s is the stored fp16 row.  A partial row is
// D fp16 values, read 8 at a time (16 bytes) by D/8 lanes, so one wave-wide
// load covers SPI = 512/D splits; the loads of all RB rows (up to BATCH per
// row, enough for 8 * SPI splits) and their (lse, e) pairs are in flight
// before any is used.  Every split slot holds a pair for every row (lse =
// -inf for a split that saw no key of the row's request), and partial rows
// of zero-weight splits may hold stale data: a select excludes them.  The
// additions run in increasing split order in every lane and do not depend
// on RB, so every caller of this function gets the same bits.
// ---------------------------------------------------------------------------
template <int D, int RB>
__device__ __forceinline__ void merge_rows_rb(const FwdParams &p, const int64_t (&r0)[RB], const bool (&on)[RB],
                                              int lane)
{
    constexpr int LPS = D / 8;       // lanes per partial row
    constexpr int SPI = 64 / LPS;    // partial rows per wave-wide load
    constexpr int BATCH = 8;         // loads per lane per row in flight
    const int ns = p.nsplit;
    const int64_t split_stride = (int64_t)p.N * p.Hq;   // rows between splits
    const int grp = lane / LPS;
    const int dcol = (lane % LPS) * 8;
    auto load = [&](int r, int s) {
        const uint16_t *src = p.ws_o + (r0[r] + (int64_t)min(s, ns - 1) * split_stride) * D + dcol;
        return *(const __attribute__((address_space(1))) f16x8 *)src;
    };
    f16x8 v[RB][BATCH];
    float ls[RB];
    int ex[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (!on[r])
            continue;
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            if (i * SPI < ns)
                v[r][i] = load(r, i * SPI + grp);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        ls[r] = -INFINITY;
        ex[r] = 0;
        if (on[r] && lane < ns) {
            const f32x2 m = gmem((const f32x2 *)p.ws_ml)[lane * split_stride + r0[r]];
            ls[r] = m[0];
            ex[r] = (int)m[1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    auto fmax_op = [](float a, float b) { return fmaxf(a, b); };
    auto add_op = [](float a, float b) { return a + b; };
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (!on[r])
            continue;
        const float mx = wave_reduce(ls[r], fmax_op);
        const float base = (mx == -INFINITY) ? 0.f : mx;
        const float wgt = (lane < ns) ? fast_exp2(ls[r] - base) : 0.f;
        const float tot = wave_reduce(wgt, add_op);
        const float wo = __builtin_ldexpf(wgt, ex[r]);   // weight of the stored (scaled) row
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto add = [&](const f16x8 &x, int s) {
            const float ws = __shfl(wo, s & 63);
            if (s < ns && ws > 0.f) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] += ws * (float)x[j];
            }
        };
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            if (i * SPI < ns)
                add(v[r][i], i * SPI + grp);
        for (int s0 = BATCH * SPI; s0 < ns; s0 += BATCH * SPI) {
            f16x8 w[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i)
                if (s0 + i * SPI < ns)
                    w[i] = load(r, s0 + i * SPI + grp);
#pragma unroll
            for (int i = 0; i < BATCH; ++i)
                if (s0 + i * SPI < ns)
                    add(w[i], s0 + i * SPI + grp);
        }
        // the LPS-lane groups hold the same columns of different splits
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (LPS <= 8)
                acc[j] += __shfl_xor(acc[j], 8);
            acc[j] = xor16(acc[j], add_op);
            acc[j] = xor32(acc[j], add_op);
        }
        if (grp == 0) {
            const float inv = tot > 0.f ? 1.0f / tot : 0.f;
            u32x4 w4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const __bf16 e0 = (__bf16)(acc[2 * j] * inv);
                const __bf16 e1 = (__bf16)(acc[2 * j + 1] * inv);
                w4[j] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
            }
            *(__attribute__((address_space(1))) u32x4 *)(gmem((uint16_t *)p.out) + r0[r] * D + dcol) = w4;
        }
        if (lane == 0)
            gmem(p.lse)[r0[r]] = tot > 0.f ? (base + __builtin_log2f(tot)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// bf16 forward: D = head dim, NW = waves per workgroup (32 query rows each)
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16): S^T = K Q^T with K as the A
// operand (LDS) and Q^T as the B operand (registers, loaded once), so a lane's
// 16 accumulators are 16 keys of ONE query row (row = lane % 32; the other 16
// keys of the 32-key tile sit in lane + 32).  Row max / sum need one
// cross-half exchange per block, and the probabilities already sit where the
// B operand of O^T = V^T P^T wants them (same lane, keys along registers).
//
// K and V blocks of 64 keys stream from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging), double-buffered, in their
// natural [key][d] layout.  Rows are XOR-swizzled in 16-byte units so the
// operand reads are free of bank conflicts: K with ds_read_b128, V^T with two
// ds_read_b64_tr_b16 (the gfx950 LDS transpose read) aimed at the exact keys
// the accumulator layout holds.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

template <int D>
struct Layout {
    static constexpr int ROWB = 2 * D;             // bytes per key row
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int BLK = 64 * ROWB;          // bytes per 64-key block
    static constexpr int RPI = 1024 / ROWB;        // rows per wave DMA instruction
    static constexpr int NINST = 64 / RPI;         // DMA instructions per block per tensor
    // physical 16-byte position of logical chunk c of row r (an involution)
    __device__ static __forceinline__ int swz_k(int r, int c)
    {
        return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    }
    __device__ static __forceinline__ int swz_v(int r, int c)
    {
        return D == 128 ? (c ^ ((r & 3) << 2)) : (c ^ (((r >> 1) & 1) << 2));
    }
};

template <int S>
struct StageTag {
    static constexpr int value = S;
};

// One wave-wide global -> LDS copy of 16 bytes per lane: lane l's bytes land
// at LDS byte address lds + 16 * l.  Issued as inline asm so that the
// compiler neither reorders LDS accesses around it nor inserts its own
// conservative waits; the kernel waits for it explicitly (TA_WAIT_VMCNT).
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

// The same copy addressed as a wave-uniform 64-bit base (scalar registers)
// plus a per-lane 32-bit byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds)
{
    // the base is uniform; read it from lane 0 so that it is certain to sit
    // in scalar registers whatever the register allocator did with it
    // (readfirstlane returns a signed int: widen through uint32_t so that the
    // low half is not sign-extended into the high half)
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(bs), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}


// Workgroup shape: NR row tiles of 32 query rows, each computed by KS waves
// that split the keys of a step between them (NW = NR * KS waves):
//   KS = 1: a step is one 64-key block; each wave computes both 32-key tiles
//   KS = 2: a step is one block; wave slice ks computes tile ks
//   KS = 4: a step is two blocks; wave slice ks computes tile ks % 2 of the
//           step's block ks / 2
// Slices of a row tile keep their own running max / sum / output and combine
// them through LDS at the end.  Key slices cut the per-wave copy, MFMA and
// store work for small row counts, where one or two waves would otherwise
// serialise a block's copy issue and math.
// SP: pages hold >= 16 tokens, so a 64-key block spans at most 4 pages whose
// ids are fetched with scalar loads; otherwise each lane loads its own.
// NSTG: K/V stages in LDS; a step's copies are issued NSTG - 1 steps ahead.
// Four stages (one key slice only) need 128 KiB at head_dim 128, so one
// workgroup per CU.
template <int D, int NR, int KS, bool SP, int NSTG>
__global__ __launch_bounds__(NR * KS * 64) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParams p_arg)
{
    const FwdParams p = load_args(p_arg);
    // K/V bases as standalone values: a select between two fields of p would
    // otherwise become a load through a selected address, which pins p in
    // scratch memory
    const char *kt_p = (const char *)p.k_tree, *vt_p = (const char *)p.v_tree;
    const char *kc_p = (const char *)p.k_cache, *vc_p = (const char *)p.v_cache;
    asm volatile("" : "+s"(kt_p), "+s"(vt_p), "+s"(kc_p), "+s"(vc_p));
    using LY = Layout<D>;
    constexpr int NW = NR * KS;
    constexpr int KSB = KS == 4 ? 2 : 1;         // 64-key blocks per step
    constexpr int NT = KS == 1 ? 2 : 1;          // 32-key tiles per wave per step
    constexpr int NKC = D / 16;                  // k steps of S^T = K Q^T
    constexpr int NDT = D / 32;                  // 32-wide d tiles of O^T
    constexpr int NI = KSB * LY::NINST;          // DMA instructions per step per tensor
    constexpr int NIW = NI / NW;                 // ... per wave
    constexpr int SBYTES = KSB * LY::BLK;        // one stage of K (or of V)
    static_assert(NI % NW == 0 && NIW >= 1, "waves must divide the DMA instructions of a step");
    static_assert(NW % KSB == 0, "a wave's DMA instructions must fall in one block");
    static_assert(NDT % KS == 0, "key slices must divide the output d tiles");
    // with more than two stages every wave issues every step's copies (one
    // key slice), which the exact copy count waited for at a step relies on
    static_assert(NSTG == 2 || (NSTG == 4 && KS == 1), "stage counts: 2, or 4 with one key slice");

    // NSTG stages of K and V (stage s: K at 2 s, V at 2 s + 1, in units of
    // SBYTES); after the key loop the same memory holds the key slices'
    // partial outputs for the combine
    __shared__ __attribute__((aligned(1024))) char kv_lds[2 * NSTG * SBYTES];
    // running (max, sum) of every slice's rows, for the final combine, and
    // the largest magnitude of each slice's share of a partial row
    __shared__ float2 ml_x[KS > 1 ? NR * KS * 32 : 1];
    __shared__ float am_x[KS > 1 ? NR * KS * 32 : 1];
    // the request's parents and first bad node, when the plan is built here
    __shared__ int32_t par_l[kMaxTree];
    __shared__ int32_t first_bad_l;
    // one word per wave for each of the two workgroup-wide ORs below
    __shared__ uint32_t red_l[2][NW];

    Unit u;
    if (!decode_unit(p, u))
        return;
    const int32_t *bt = p.block_table + (int64_t)u.b * p.max_pages;
    typedef const __attribute__((address_space(4))) int32_t *cint_p;
    // the block table is read-only for the whole launch: read it through the
    // constant address space so that page ids come in with scalar loads
    const cint_p btc = (cint_p)bt;
    // Page ids of the split's first step depend on the split alone, so they
    // are read together with the request geometry (one memory round trip).
    // Without a block table the loads read prefix_len[0] instead (unused).
    int pg0[4 * KSB];
    if (SP) {
        const bool have = p.max_pages > 0;
        const cint_p src = have ? btc : (cint_p)p.prefix_len;
        const int pf = (u.s * p.chunk) >> p.page_shift;
#pragma unroll
        for (int q = 0; q < 4 * KSB; ++q)
            pg0[q] = src[have ? min(pf + q, p.max_pages - 1) : 0];
    }
    const ReqInfo R = request_info(p, u.b, u.s);
    if (SP) {
        // both sets of loads in flight before either is waited for (the
        // compiler would otherwise sink the page-id loads past the exits)
#pragma unroll
        for (int q = 0; q < 4 * KSB; ++q)
            asm volatile("" : "+s"(pg0[q]));
    }
    // With a parent array the units that own a request's tree also build its
    // plan.  The request-level checks come first, on the raw geometry, with
    // the plan's status codes.
    const bool fuse = p.parent != nullptr;
    int req_status = kTreeOk;
    int L_raw = 0;
    if (fuse && R.owns_tree) {
        const int off_raw = ((cint_p)p.tree_off)[u.b];
        const int end_raw = ((cint_p)p.tree_off)[u.b + 1];
        L_raw = ((cint_p)p.prefix_len)[u.b];
        const int T_raw = end_raw - off_raw;
        const bool bad_off = T_raw < 0 || T_raw > p.max_tree || off_raw < 0 || end_raw > p.N ||
                             (u.b == 0 && off_raw != 0) || (u.b == p.B - 1 && end_raw != p.N);
        req_status = bad_off ? kTreeBadOffsets : (L_raw < 0 ? kTreeBadPrefix : kTreeOk);
    }
    const int rows = R.T * p.G;
    const int row0 = u.rt * (NR * 32);
    if (row0 >= rows) {
        // an empty tree (or one whose clamped size is 0) still gets a status
        if (fuse && R.owns_tree && u.c == 0 && u.rt == 0 && threadIdx.x == 0)
            gmem(p.plan_status)[u.b] = req_status;
        return;   // uniform across the workgroup
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave; saying so lets everything
    // derived from it (DMA rows, page choices, LDS bases) live in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rtw = wv % NR;    // the wave's row tile
    const int ks = wv / NR;     // the wave's key slice
    const int hh = lane >> 5;   // which half of the wave
    const int lr = lane & 31;   // query row inside the wave's tile
    const int my_row = row0 + rtw * 32 + lr;
    const bool row_ok = my_row < rows;
    const int node = row_ok ? my_row / p.G : 0;
    const int qh = u.c * p.G + (row_ok ? my_row - node * p.G : 0);
    if (!R.owns_tree && R.kend <= R.kstart) {
        // an empty prefix split (past its request's prefix): its rows'
        // partial lse is -inf, so the merge gives it zero weight and never
        // reads its partial output
        if (row_ok && hh == 0 && ks == 0)
            store_through(&gmem((f32x2 *)p.ws_ml)[((int64_t)u.s * p.N + R.off + node) * p.Hq + qh], __builtin_bit_cast(u32x2, f32x2{-INFINITY, 0.f}));
        return;   // uniform across the workgroup
    }
    const int c = u.c;
    const int64_t head_off = (int64_t)c * D;
    const int64_t row_stride = (int64_t)p.Hkv * D;   // elements between key rows
    const int pmask = (1 << p.page_shift) - 1;

    const int n_pre = (R.kend - R.kstart + 63) / 64;
    int tree_need = 0;

    // block k -> (is_tree, first key): prefix blocks first, then tree blocks
    auto block_start = [&](int k, bool &is_tree) -> int {
        if (k < n_pre) {
            is_tree = false;
            return R.kstart + k * 64;
        }
        int m = tree_need;
        for (int i = k - n_pre; i > 0; --i)
            m &= m - 1;
        is_tree = true;
        return __builtin_ctz(m) * 64;
    };

    // This wave's DMA instructions of a step: instruction gi = wv * NIW + i
    // covers rows (gi % NINST) * RPI .. +RPI of the step's block gi / NINST
    // (the same block for all i); the lane's 16 bytes go to position
    // lane % CPR of its row.
    const int dma_blk = (wv * NIW) / LY::NINST;
    int dma_row[NIW];
#pragma unroll
    for (int i = 0; i < NIW; ++i)
        dma_row[i] = ((wv * NIW + i) % LY::NINST) * LY::RPI + lane / LY::CPR;
    const int dma_pos = lane % LY::CPR;
    // SP prefix copies: an instruction's RPI rows lie in one page (pages hold
    // >= 16 tokens, instructions start at multiples of RPI <= 16), so its
    // source is a uniform page row plus this lane's constant byte offset
    // (row inside the instruction, kv head, swizzled 16-byte chunk).
    const int64_t row_bytes = row_stride * 2;   // bytes between consecutive key rows
    const int lrow = lane / LY::CPR;                      // row inside an instruction
    const uint32_t lrow_b = (uint32_t)(lrow * row_bytes);
    uint32_t kofs[NIW], vofs[NIW];
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
        const uint32_t rb = lrow_b + (uint32_t)(head_off * 2);
        kofs[i] = rb + LY::swz_k(dma_row[i], dma_pos) * 16;
        vofs[i] = rb + LY::swz_v(dma_row[i], dma_pos) * 16;
    }

    // Full prefix blocks (SP): the wave's rows [wrow0, wrow0 + NIW * RPI)
    // fall in GPW groups of 16 rows, each inside one page.  The page id of
    // every group is read one step ahead (pf_pg, scalar loads that complete
    // during the step in between), and each group's rows are addressed from
    // one uniform base: the row inside the group moves into the lane's
    // constant offset.
    constexpr int WROWS = NIW * LY::RPI;                  // rows per wave per step
    constexpr int GPW = WROWS >= 16 ? WROWS / 16 : 1;     // 16-row groups per wave
    const int wrow0 = ((wv * NIW) % LY::NINST) * LY::RPI; // the wave's first row in its block
    const int grp0 = wrow0 & ~15;                         // first row of its first group
    uint32_t kofs_g[NIW], vofs_g[NIW];
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
        const uint32_t in_grp = (uint32_t)((wrow0 + i * LY::RPI - grp0) & 15) * (uint32_t)row_bytes;
        kofs_g[i] = kofs[i] + in_grp;
        vofs_g[i] = vofs[i] + in_grp;
    }
    int pf_pg[GPW];
#pragma unroll
    for (int g = 0; g < GPW; ++g)
        pf_pg[g] = 0;
    // page ids of step j's groups, for a later non-first issue of step j
    auto prefetch_pages = [&](int j) __attribute__((always_inline)) {
        if (!SP)
            return;
        const int k = j * KSB + dma_blk;
        if (k >= n_pre)
            return;
        const int t0 = R.kstart + k * 64 + grp0;
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            const int t = t0 + g * 16;
            pf_pg[g] = t < R.kend ? btc[t >> p.page_shift] : 0;
        }
    };

    // Issue this wave's copies of step j into a stage.  Page ids never come
    // from vector loads left in flight (the loop's vmcnt waits count DMA
    // instructions only): with SP a full block uses the ids prefetched a step
    // ahead (pf_pg), the split's first step those read into pg0, and a ragged
    // block scalar loads; smaller pages use per-lane loads, consumed before
    // the DMA is issued.
    // FIRST: the split's first step, whose page ids were read into pg0
    auto issue_dma = [&](int j, auto stage, auto first) {
        constexpr bool FIRST = decltype(first)::value != 0;
        const int k = j * KSB + dma_blk;
        if (k >= (n_pre + __builtin_popcount(tree_need)))
            return;
        bool is_tree;
        const int start = block_start(k, is_tree);
        char *kst = kv_lds + 2 * decltype(stage)::value * SBYTES + dma_blk * LY::BLK;
        char *vst = kst + SBYTES;
        const uint16_t *kb = (const uint16_t *)(is_tree ? kt_p : kc_p);
        const uint16_t *vb = (const uint16_t *)(is_tree ? vt_p : vc_p);
        if (SP && !is_tree && !FIRST && start + 64 <= R.kend) {
            // a full prefix block whose group page ids were prefetched
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                int page = pf_pg[g];
                page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
                const int tg = start + grp0 + g * 16;   // the group's first key
                const int64_t gb = (((int64_t)page << p.page_shift) + (tg & pmask)) * row_bytes;
#pragma unroll
                for (int i = 0; i < NIW; ++i) {
                    if (((wrow0 + i * LY::RPI - grp0) >> 4) != g)
                        continue;   // compile-time for a given wave shape
                    const int gl = (wv * NIW + i) % LY::NINST;
                    const uint32_t ldsk = __builtin_amdgcn_readfirstlane(lds_addr(kst) + gl * 1024);
                    const uint32_t ldsv = __builtin_amdgcn_readfirstlane(lds_addr(vst) + gl * 1024);
                    dma16s(kc_p + gb, kofs_g[i], ldsk);
                    dma16s(vc_p + gb, vofs_g[i], ldsv);
                }
            }
            return;
        }
        int pages[4] = {0, 0, 0, 0};
        const int pfirst = __builtin_amdgcn_readfirstlane(start >> p.page_shift);
        if (SP && !is_tree) {
            if (FIRST) {
                // pg0[i] is the page of key (split start) + i * page_size
                const int rel = pfirst - ((u.s * p.chunk) >> p.page_shift);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int v = 0;
#pragma unroll
                    for (int i = 0; i < 4 * KSB; ++i)
                        v = (i == rel + q) ? pg0[i] : v;
                    pages[q] = v;
                }
            } else {
                const int last = min(start + 63, R.kend - 1);
                const int plast = __builtin_amdgcn_readfirstlane(last >> p.page_shift);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pages[q] = (pfirst + q <= plast) ? btc[pfirst + q] : 0;
            }
        }
        if (SP && !is_tree) {
            // Keys at or past kend are masked, but their rows must still hold
            // finite values (0 * NaN in P V would poison the output), so in
            // the ragged last block they are read from a valid key instead:
            // the instruction's first row, or the block's first key when the
            // whole instruction lies past kend.
            const bool ragged = start + 64 > R.kend;   // uniform
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int gl = (wv * NIW + i) % LY::NINST;
                int t0 = start + gl * LY::RPI;           // first key of the instruction's rows
                uint32_t ko = kofs[i], vo = vofs[i];
                if (ragged) {
                    if (t0 >= R.kend) {
                        t0 = start;
                        ko -= lrow_b;
                        vo -= lrow_b;
                    } else if (t0 + lrow >= R.kend) {
                        ko -= lrow_b;
                        vo -= lrow_b;
                    }
                }
                const int q = (t0 >> p.page_shift) - pfirst;
                int page = q == 0 ? pages[0] : (q == 1 ? pages[1] : (q == 2 ? pages[2] : pages[3]));
                page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
                page = __builtin_amdgcn_readfirstlane(page);   // uniform by construction
                const int64_t rowo = (((int64_t)page << p.page_shift) + (t0 & pmask)) * row_bytes;
                const uint32_t ldsk = __builtin_amdgcn_readfirstlane(lds_addr(kst) + gl * 1024);
                const uint32_t ldsv = __builtin_amdgcn_readfirstlane(lds_addr(vst) + gl * 1024);
                dma16s(kc_p + rowo, ko, ldsk);
                dma16s(vc_p + rowo, vo, ldsv);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < NIW; ++i) {
            const int r = dma_row[i];
            int64_t off;
            if (is_tree) {
                int jn = start + r;
                jn = jn < R.T ? jn : start;   // rows past the tree: a valid, masked row
                off = (int64_t)(R.off + jn) * row_stride + head_off;
            } else {
                int t = start + r;
                t = t < R.kend ? t : start;   // keys past the split: a valid, masked row
                int page;
                if (SP) {
                    const int q = (t >> p.page_shift) - pfirst;
                    page = q == 0 ? pages[0] : (q == 1 ? pages[1] : (q == 2 ? pages[2] : pages[3]));
                } else {
                    page = gmem(bt)[t >> p.page_shift];
                }
                page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
                off = (((int64_t)page << p.page_shift) + (t & pmask)) * row_stride + head_off;
            }
            const int gl = (wv * NIW + i) % LY::NINST;
            const int ck = LY::swz_k(r, dma_pos);
            const int cv = LY::swz_v(r, dma_pos);
            dma16(kb + off + ck * 8, __builtin_amdgcn_readfirstlane(lds_addr(kst) + gl * 1024));
            dma16(vb + off + cv * 8, __builtin_amdgcn_readfirstlane(lds_addr(vst) + gl * 1024));
        }
    };

    // Q^T fragments (B operand): lane holds Q[row][kc*16 + hh*8 .. +8].
    // Issued first: a wave's copy instructions below take about 116 clocks
    // each to issue, and behind them the Q loads went out late (budget 16,
    // one request: attention kernel 9.32 -> 9.03 us with Q first).
    bf16x8 qf[NKC];
    {
        const auto qrow = gmem((const uint16_t *)p.q + ((int64_t)(R.off + node) * p.Hq + qh) * D);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok)
                v = *(const __attribute__((address_space(1))) u32x4 *)(qrow + kc * 16 + hh * 8);
            qf[kc] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // The split's first prefix step is copied right after the Q loads and
    // before the mask words are loaded, so the three travel together.
    // (a unit that owns the tree copies early only a step of prefix blocks:
    // which tree blocks it needs is known after the mask words arrive)
    const bool early = SP && n_pre > 0 && (n_pre >= KSB || !R.owns_tree);
    if (early) {
        // pg0 holds the pages from the split's first key on; rows past kend
        // fall back to the block's first key, so only valid pages are used
        issue_dma(0, StageTag<0>(), StageTag<1>());
        prefetch_pages(1);
    }
    // A tree-only unit of a request whose tree fits one 64-node block needs
    // that block whatever the mask words say (every row sees its own node),
    // so its copy starts here too, before the mask words (or the parents)
    // are read.
    const bool early_tree = R.owns_tree && n_pre == 0 && R.T <= 64;
    if (early_tree) {
        tree_need = 1;
        issue_dma(0, StageTag<0>(), StageTag<0>());
    }

    // tree blocks this workgroup needs (only the unit that owns the tree)
    // OR of four per-lane flag bits over the workgroup: a ballot per bit in
    // each wave, one LDS word per wave, one barrier (slot: which of the two
    // uses, each made once)
    auto block_or4 = [&](uint32_t bits, int slot) __attribute__((always_inline)) -> uint32_t {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            v |= (__ballot((bits >> b) & 1u) != 0ull) ? (1u << b) : 0u;
        if (lane == 0)
            red_l[slot][wv] = v;
        __syncthreads();
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            r |= red_l[slot][w];
        return r;
    };

    uint64_t mw[kMaskWords] = {0, 0, 0, 0};
    if (R.owns_tree && fuse && R.T <= 64) {
        // The plan of a tree of up to 64 nodes, in every wave on its own (no
        // workgroup barrier): lane l loads node l's parent, a ballot finds the
        // first bad parent (parent[j] outside [-1, j)), and the ancestor sets
        // come by pointer jumping.  Lane l holds the nodes from l up to, not
        // including, jp (its first ancestor not yet merged); each round merges
        // jp's set and jumps to jp's jp, so a path of depth d needs about
        // log2(d) rounds of cross-lane reads where walking it costs d
        // dependent loads.  Each row then takes its node's word from the lane
        // that holds it.  Units of kv head 0 write the plan's outputs: one
        // row per node (its group's first q head) and, from row tile 0, the
        // request's status.
        int jp = -1;
        if (req_status == kTreeOk && lane < R.T)
            jp = gmem(p.parent)[R.off + lane];
        const uint64_t bad = __ballot(lane < R.T && (jp < -1 || jp >= lane));
        if (req_status == kTreeOk && bad != 0ull)
            req_status = __builtin_ctzll(bad) + 1;   // uniform: every wave reads the same parents
        if (req_status == kTreeOk) {
            uint64_t m = lane < R.T ? (1ull << lane) : 0ull;
            while (__ballot(jp >= 0) != 0ull) {      // ends: parents precede children
                const int src = jp >= 0 ? jp : lane;
                const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)m, src);
                const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(m >> 32), src);
                const int jj = __shfl(jp, src);
                if (jp >= 0) {
                    m |= ((uint64_t)hi << 32) | lo;
                    jp = jj;
                }
            }
            const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)m, node);
            const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(m >> 32), node);
            const uint64_t wrow = ((uint64_t)hi << 32) | lo;
            if (row_ok) {
                mw[0] = wrow;
                if (c == 0 && hh == 0 && ks == 0 && my_row == node * p.G) {
                    const int64_t n = R.off + node;
                    const int d = __builtin_popcountll(wrow);
                    const auto mrow = gmem(p.plan_mask) + n * kMaskWords;
                    mrow[0] = wrow;
                    mrow[1] = 0ull;
                    mrow[2] = 0ull;
                    mrow[3] = 0ull;
                    gmem(p.plan_depth)[n] = d;
                    gmem(p.plan_pos)[n] = L_raw + d - 1;
                }
            }
            // every row sees its own node, all in the first 64-node block
            tree_need |= 1;
        }
        if (c == 0 && u.rt == 0 && tid == 0)
            gmem(p.plan_status)[u.b] = req_status;
    } else if (R.owns_tree) {
        if (fuse) {
            // Larger trees: stage the request's parents in LDS and check them
            // as the plan does (parent[j] in [-1, j)); then each row walks its
            // node's parent chain, which ends within node + 1 steps.  Outputs
            // as above.
            constexpr int NPT = (kMaxTree + NW * 64 - 1) / (NW * 64);   // parents per thread
            uint32_t badp = 0;
            if (req_status == kTreeOk) {
                const auto pg = gmem(p.parent) + R.off;
                int pj[NPT];
#pragma unroll
                for (int i = 0; i < NPT; ++i) {
                    const int j = tid + i * NW * 64;
                    pj[i] = j < R.T ? pg[j] : -1;
                }
#pragma unroll
                for (int i = 0; i < NPT; ++i) {
                    const int j = tid + i * NW * 64;
                    if (j < R.T) {
                        par_l[j] = pj[i];
                        badp |= (pj[i] < -1 || pj[i] >= j) ? 1u : 0u;
                    }
                }
            }
            if (block_or4(badp, 0)) {
                if (tid == 0)
                    first_bad_l = INT32_MAX;
                __syncthreads();
                for (int j = tid; j < R.T; j += NW * 64) {
                    const int pj = par_l[j];
                    if (pj < -1 || pj >= j)
                        atomicMin(&first_bad_l, j);
                }
                __syncthreads();
                req_status = first_bad_l + 1;
            }
            if (req_status == kTreeOk && row_ok) {
                uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
                int d = 0;
                for (int a = node; a >= 0; a = par_l[a]) {
                    const uint64_t bit = 1ull << (a & 63);
                    const int word = a >> 6;
                    w0 |= word == 0 ? bit : 0ull;
                    w1 |= word == 1 ? bit : 0ull;
                    w2 |= word == 2 ? bit : 0ull;
                    w3 |= word == 3 ? bit : 0ull;
                    ++d;
                }
                mw[0] = w0;
                mw[1] = w1;
                mw[2] = w2;
                mw[3] = w3;
                if (c == 0 && hh == 0 && ks == 0 && my_row == node * p.G) {
                    const int64_t n = R.off + node;
                    const auto mrow = gmem(p.plan_mask) + n * kMaskWords;
                    mrow[0] = w0;
                    mrow[1] = w1;
                    mrow[2] = w2;
                    mrow[3] = w3;
                    gmem(p.plan_depth)[n] = d;
                    gmem(p.plan_pos)[n] = L_raw + d - 1;
                }
            }
            if (c == 0 && u.rt == 0 && tid == 0)
                gmem(p.plan_status)[u.b] = req_status;
        } else if (row_ok) {
            const auto mrow = gmem(p.anc_mask + (int64_t)(R.off + node) * kMaskWords);
#pragma unroll
            for (int w = 0; w < kMaskWords; ++w)
                mw[w] = (w * 64 < R.T) ? mrow[w] : 0ull;
        }
        uint32_t nz = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w)
            nz |= mw[w] != 0ull ? (1u << w) : 0u;
        tree_need |= (int)block_or4(nz, 1);
    }
    const int n_blocks = n_pre + __builtin_popcount(tree_need);
    const int n_steps = (n_blocks + KSB - 1) / KSB;

    // per-lane LDS offsets of the operand reads (row parts fold into immediates)
    // K (A of S^T): row kt*32 + lr, logical chunk kc*2 + hh
    // V^T (A of O^T) through the transpose read: source lane (e, q) of its
    // 16-lane group reads 4 d-values [dcol, dcol+4) of key row
    //   kt*32 + kc*16 + half*8 + hh*4 + e,  dcol = dt*32 + ((lane/16)&1)*16 + 4q
    const int te = (lane & 15) >> 2;
    const int tq = lane & 3;
    const int v_row_l = hh * 4 + te;                         // row part owned by the lane
    const int v_chunk_l = ((lane >> 4) & 1) * 2 + (tq >> 1);  // chunk within a 32-wide d tile
    const int v_half = (tq & 1) * 8;                          // byte offset inside the chunk
    const int my_blk = KS == 4 ? (ks >> 1) : 0;              // the wave's block in a step

    f32x16 acc_o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        acc_o[dt] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max, scaled log2 domain
    float l_run = 0.f;         // this half's partial sum of probabilities
    const float c2 = p.c2;

    // one step: wait for this step's DMA, one barrier (every wave's copy has
    // landed and every wave has finished the step before), start the DMA of
    // step j + NSTG - 1 into the stage read in step j - 1, then the math on
    // this stage.  One barrier per step suffices because a stage is refilled
    // only after it.
    auto step = [&](int j, auto stage) {
        if constexpr (NSTG == 2) {
            TA_WAIT_VMCNT(0);                   // this wave's step-j DMA has landed
        } else {
            // The copies of steps j + 1 .. j + NSTG - 2 (those below n_steps,
            // 2 NIW instructions each) may stay in flight: copies complete
            // in issue order, so then step j's have landed.  A vector load
            // of the compiler's own issued in between only makes this wait
            // stricter.
            static_assert(NSTG == 4, "the waits below are written for four stages");
            const int ahead = n_steps - 1 - j;
            if (ahead >= 2)
                TA_WAIT_VMCNT(4 * NIW);
            else if (ahead == 1)
                TA_WAIT_VMCNT(2 * NIW);
            else
                TA_WAIT_VMCNT(0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): its LDS reads of step j-1 are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();           // ... and every other wave's too
        asm volatile("" ::: "memory");          // no LDS access moves across it
        if (j + NSTG - 1 < n_steps) {
            // that stage was last read in step j-1, which every wave has left
            issue_dma(j + NSTG - 1, StageTag<(decltype(stage)::value + NSTG - 1) % NSTG>(), StageTag<0>());
            prefetch_pages(j + NSTG);
        }
        const int k = j * KSB + my_blk;
        if (k < n_blocks) {
            bool is_tree;
            const int start = block_start(k, is_tree);
            const char *kst = kv_lds + 2 * decltype(stage)::value * SBYTES + my_blk * LY::BLK;
            const char *vst = kst + SBYTES;

            // which 32-key tiles of the block this wave computes
            int ktile[NT];
            bool active[NT];
            uint32_t bits[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                ktile[t] = KS == 1 ? t : (ks & 1);
                bits[t] = 0xffffffffu;
            }
            if (is_tree) {
                const int w = start >> 6;
                uint64_t word = 0;
#pragma unroll
                for (int i = 0; i < kMaskWords; ++i)
                    word = (i == w) ? mw[i] : word;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    bits[t] = ktile[t] ? (uint32_t)(word >> 32) : (uint32_t)word;
                    active[t] = __ballot(bits[t] != 0u) != 0ull;
                }
            } else {
                const int valid = R.kend - start;   // keys of this block inside the split
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int vt = valid - ktile[t] * 32;   // keys of this tile inside the split
                    active[t] = vt > 0;
                    if (vt < 32)
                        bits[t] = vt <= 0 ? 0u : ((1u << vt) - 1u);
                }
            }
            const bool masked = is_tree || (start + 64 > R.kend);

            // the first MFMA of a tile takes the zero accumulator as an inline
            // constant, so no register is cleared per block
            const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            f32x16 s_acc[NT];
            // With two tiles per wave both are computed whatever their mask
            // (an inactive tile's scores are masked to -inf below, and its
            // K rows are finite), so that the two MFMA chains share one basic
            // block; a lone tile is skipped when no row sees it.
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (NT > 1 || active[t]) {
                    const int r = ktile[t] * 32 + lr;
                    const char *krow = kst + r * LY::ROWB;
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc) {
                        const bf16x8 a = *(const bf16x8 *)(krow + LY::swz_k(r, kc * 2 + hh) * 16);
                        s_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], kc == 0 ? zero16 : s_acc[t], 0, 0, 0);
                    }
                } else {
                    s_acc[t] = zero16;
                }
            }
            if constexpr (NT > 1) {
                // K reads kept four ahead of the MFMAs that use them
                // (masks: 0x100 LDS read, 0x008 MFMA)
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 2 * NKC - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            if (masked) {
                // lane value i of a tile is key tile*32 + (i/4)*8 + hh*4 + i%4
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint32_t bk = active[t] ? (bits[t] >> (hh * 4)) : 0u;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kk = (i >> 2) * 8 + (i & 3);
                        s_acc[t][i] = ((bk >> kk) & 1u) ? s_acc[t][i] : -INFINITY;
                    }
                }
            }

            // online softmax
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, s_acc[t][i]);
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
            for (int t = 0; t < NT; ++t) {
                // as for S: with two tiles an inactive one runs too (its
                // probabilities are 0 and its V rows finite), keeping both
                // tiles' exponentials and P V in one basic block
                if (NT == 1 && !active[t])
                    continue;
                bf16x8 pb[2];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    pb[i >> 3][i & 7] = (__bf16)fast_exp2(__builtin_fmaf(s_acc[t][i], c2, -mu));
                // The row sum adds the bf16 probabilities the PV product uses
                // (numerator and denominator share the same weights), two per
                // v_dot2_f32_bf16 against (1, 1).
                const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
                float ls[2] = {0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bf16x2 pr = {pb[j >> 2][(2 * j) & 7], pb[j >> 2][(2 * j + 1) & 7]};
                    ls[j & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls[j & 1], false);
                }
                l_run += ls[0] + ls[1];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const int rbase = ktile[t] * 32 + kc * 16 + v_row_l;   // half 0; half 1 is +8
                    const char *v0 = vst + rbase * LY::ROWB + v_half;
                    const char *v1 = v0 + 8 * LY::ROWB;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        // rows rbase and rbase + 8 share the swizzle
                        const int pos = LY::swz_v(rbase, dt * 4 + v_chunk_l) * 16;
                        typedef short i16x4 __attribute__((ext_vector_type(4)));
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(v0 + pos));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(v1 + pos));
                        typedef short i16x8 __attribute__((ext_vector_type(8)));
                        const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
                        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], acc_o[dt], 0, 0, 0);
                    }
                }
            }
        }
    };

    // Q and mask words are in registers before the loop: the compiler,
    // which does not see the DMA, then has no load of its own outstanding
    // inside the loop and inserts no waits there.
    TA_WAIT_VMCNT(0);
    if (!early && !early_tree && n_steps > 0) {
        prefetch_pages(0);
        issue_dma(0, StageTag<0>(), StageTag<0>());
        prefetch_pages(1);
    }
    if constexpr (NSTG == 4) {
        // steps 1 and 2 go out before the loop, each with the page ids
        // prefetched just before it
        if (1 < n_steps) {
            issue_dma(1, StageTag<1>(), StageTag<0>());
            prefetch_pages(2);
        }
        if (2 < n_steps) {
            issue_dma(2, StageTag<2>(), StageTag<0>());
            prefetch_pages(3);
        }
    }
    for (int j = 0; j < n_steps; j += NSTG) {
        step(j, StageTag<0>());
        if (j + 1 < n_steps)
            step(j + 1, StageTag<1>());
        if constexpr (NSTG == 4) {
            if (j + 2 < n_steps)
                step(j + 2, StageTag<2>());
            if (j + 3 < n_steps)
                step(j + 3, StageTag<3>());
        }
    }
    if (KS > 1) {
        // the slice combine below reuses the stages: every wave must be done
        // reading them
        __builtin_amdgcn_s_waitcnt(0xc07f);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    float l_tot = l_run + __shfl_xor(l_run, 32);
    float m_fin = m_run;
    // d tiles this wave writes: all with one slice, else those with dt % KS == ks
    auto owns_dt = [&](int dt) { return KS == 1 || (dt % KS) == ks; };
    if (KS > 1) {
        // Combine the key slices of each row tile.  Every wave publishes its
        // rows' (max, sum) and the output tiles it does not own; the stages
        // are free after the barrier above.
        float *xo = (float *)kv_lds;   // [NR][KS][NDT - NDT/KS][32 x 32] fp32, lane-major
        constexpr int NX = NDT - NDT / KS;
        static_assert(NR * KS * NX * 4096 <= 2 * NSTG * SBYTES, "combine buffer exceeds the stages");
        if (hh == 0)
            ml_x[(rtw * KS + ks) * 32 + lr] = float2{m_run, l_tot};
        int x = 0;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (owns_dt(dt))
                continue;
            float4 *dst = (float4 *)(xo + (((rtw * KS + ks) * NX + x) * 1024));
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                dst[i4 * 64 + lane] = float4{acc_o[dt][i4 * 4 + 0], acc_o[dt][i4 * 4 + 1],
                                             acc_o[dt][i4 * 4 + 2], acc_o[dt][i4 * 4 + 3]};
            ++x;
        }
        __syncthreads();
        float mk[KS], lk[KS];
        float mall = -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const float2 v = ml_x[(rtw * KS + s2) * 32 + lr];
            mk[s2] = v.x;
            lk[s2] = v.y;
            mall = fmaxf(mall, v.x);
        }
        const float base = mall == -INFINITY ? 0.f : mall;
        float ak[KS];
        float lsum = 0.f, a_own = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            ak[s2] = mk[s2] == -INFINITY ? 0.f : fast_exp2(mk[s2] - base);
            lsum += ak[s2] * lk[s2];
            a_own = s2 == ks ? ak[s2] : a_own;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (!owns_dt(dt))
                continue;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc_o[dt][i] *= a_own;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                if (s2 == ks)
                    continue;
                // slot of dt among the tiles slice s2 does not own
                int x2 = 0;
                for (int d2 = 0; d2 < dt; ++d2)
                    x2 += (d2 % KS) != s2;
                const float4 *srcx = (const float4 *)(xo + (((rtw * KS + s2) * NX + x2) * 1024));
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 v = srcx[i4 * 64 + lane];
                    acc_o[dt][i4 * 4 + 0] += ak[s2] * v.x;
                    acc_o[dt][i4 * 4 + 1] += ak[s2] * v.y;
                    acc_o[dt][i4 * 4 + 2] += ak[s2] * v.z;
                    acc_o[dt][i4 * 4 + 3] += ak[s2] * v.w;
                }
            }
        }
        l_tot = lsum;
        m_fin = base;
    }
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_fin + __builtin_log2f(l_tot) : -INFINITY;
    const int64_t n = R.off + node;
    const bool lse_writer = hh == 0 && ks == 0;
    if (KS == 1 && NSTG == 2 && p.nsplit > 1) {
        // One slice, split partials: the rows go out through LDS.  A lane
        // holds 8 bytes of each 16-byte chunk of its row, so storing from
        // registers writes 16 bytes into each of 32 rows per instruction,
        // and the L2 sees 16-byte requests.  Each wave instead stages its 32
        // rows in a region of its own (row-major, chunks XOR-swizzled by
        // row) and stores whole rows, D/8 lanes per row.  The values are
        // converted exactly as below, so the results are the same bits
        // (budget 256, one request: step 27.4 -> 26.6 us; 8 requests of
        // budget 64: 46.1 -> 45.6 us).  Unsplit outputs keep the direct
        // stores: there the barrier and the round trip cost more (32
        // requests of budget 256: 554 -> 568 us when staged), and the
        // four-stage form, which serves that shape, does not hold this
        // code at all (with it, unused, it ran 556 -> 579 us).
        static_assert(NW * 32 * LY::ROWB <= 2 * NSTG * SBYTES, "output staging exceeds the stages");
        constexpr int CPR = LY::CPR;      // 16-byte chunks per row
        constexpr int RPS = 64 / CPR;     // rows per store instruction
        __builtin_amdgcn_s_waitcnt(0xc07f);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();     // every wave has left the last step: the stages are free
        asm volatile("" ::: "memory");
        // the partial row scaled by 2^-e (see below)
        float am = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                am = fmaxf(am, __builtin_fabsf(acc_o[dt][i]));
        am = fmaxf(am, __shfl_xor(am, 32));
        const float mo = am * inv;
        const int ex = mo > 0.f ? __builtin_amdgcn_frexp_expf(mo) - 15 : 0;
        char *const wreg = kv_lds + wv * (32 * LY::ROWB);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f16x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (_Float16)__builtin_ldexpf(acc_o[dt][i4 * 4 + j] * inv, -ex);
                const u32x2 w2 = __builtin_bit_cast(u32x2, v);
                const int q = dt * 4 + i4;   // the chunk of columns dt*32 + i4*8 .. +8
                *(u32x2 *)(wreg + lr * LY::ROWB + ((q ^ (lr & (CPR - 1))) * 16) + hh * 8) = w2;
            }
        }
        if (lse_writer && row_ok)
            store_through(&gmem((f32x2 *)p.ws_ml)[((int64_t)u.s * p.N + n) * p.Hq + qh], __builtin_bit_cast(u32x2, f32x2{lse2, (float)ex}));
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) {
            const int rr = i * RPS + lane / CPR;
            const int q = lane % CPR;
            const u32x4 v = *(const u32x4 *)(wreg + rr * LY::ROWB + ((q ^ (rr & (CPR - 1))) * 16));
            const int mr = row0 + rtw * 32 + rr;   // the row's index among the (b, c) rows
            if (mr < rows) {
                const int nd = mr / p.G;
                const int64_t nn = R.off + nd;
                const int qr = c * p.G + (mr - nd * p.G);
                uint16_t *dst = p.ws_o + (((int64_t)u.s * p.N + nn) * p.Hq + qr) * D;
                store_through(gmem(dst) + q * 8, v);
            }
        }
        return;
    }
    if (p.nsplit == 1) {
        if (!row_ok)
            return;
        const auto orow = gmem((uint16_t *)p.out + (n * p.Hq + qh) * D);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (!owns_dt(dt))
                continue;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const __bf16 e0 = (__bf16)(acc_o[dt][i4 * 4 + 0] * inv);
                const __bf16 e1 = (__bf16)(acc_o[dt][i4 * 4 + 1] * inv);
                const __bf16 e2 = (__bf16)(acc_o[dt][i4 * 4 + 2] * inv);
                const __bf16 e3 = (__bf16)(acc_o[dt][i4 * 4 + 3] * inv);
                u32x2 w2;
                w2[0] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
                w2[1] = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
                *(__attribute__((address_space(1))) u32x2 *)(orow + dt * 32 + i4 * 8 + hh * 4) = w2;
            }
        }
        if (lse_writer)
            gmem(p.lse)[n * p.Hq + qh] = lse2 * kLn2;
        return;
    }
    // A split's partial row: the normalised output scaled by 2^-e so that its
    // largest magnitude lies in [2^14, 2^15), inside the fp16 range whatever
    // the range of V, with e stored beside its lse.  Scaling by a power of
    // two changes no rounding, so the stored value is the fp16 rounding of
    // the exact normalised value, scaled.
    float am = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        if (!owns_dt(dt))
            continue;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            am = fmaxf(am, __builtin_fabsf(acc_o[dt][i]));
    }
    am = fmaxf(am, __shfl_xor(am, 32));
    if (KS > 1) {
        // the row's other columns belong to the other key slices
        if (hh == 0)
            am_x[(rtw * KS + ks) * 32 + lr] = am;
        __syncthreads();
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
            am = fmaxf(am, am_x[(rtw * KS + s2) * 32 + lr]);
    }
    const float mo = am * inv;
    const int ex = mo > 0.f ? __builtin_amdgcn_frexp_expf(mo) - 15 : 0;   // mo * 2^-ex in [2^14, 2^15)
    // Key slices: a wave owns NDT/KS column tiles (32 columns each) of its 32
    // rows.  Where the stage memory above the slice-combine buffer can hold
    // them, each wave stages its owned columns there (row-major, chunks
    // XOR-swizzled by row; the combine buffer is not touched, so no barrier
    // is needed) and stores 64-byte runs per row instead of 16 bytes into
    // each of 32 rows per instruction.  Same values, same bits (budget 16,
    // one request: step 12.62 -> 12.49 us).
    constexpr int XO_BYTES = KS > 1 ? NR * KS * (NDT - NDT / KS) * 4096 : 0;
    constexpr int CPW = (NDT / KS) * 4;   // owned 16-byte chunks per row
    constexpr bool STAGE_SLICES = KS > 1 && (CPW & (CPW - 1)) == 0 &&
                                  XO_BYTES + NW * 32 * CPW * 16 <= 2 * NSTG * SBYTES;
    if constexpr (STAGE_SLICES) {
        char *const wreg = kv_lds + XO_BYTES + wv * (32 * CPW * 16);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (!owns_dt(dt))
                continue;           // compile-time index into acc_o, runtime skip
            const int t = dt / KS;  // the owned tile's rank: dt = ks + KS t
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f16x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (_Float16)__builtin_ldexpf(acc_o[dt][i4 * 4 + j] * inv, -ex);
                const int lq = t * 4 + i4;
                *(u32x2 *)(wreg + lr * (CPW * 16) + ((lq ^ (lr & (CPW - 1))) * 16) + hh * 8) =
                    __builtin_bit_cast(u32x2, v);
            }
        }
        if (lse_writer && row_ok)
            store_through(&gmem((f32x2 *)p.ws_ml)[((int64_t)u.s * p.N + n) * p.Hq + qh], __builtin_bit_cast(u32x2, f32x2{lse2, (float)ex}));
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
        asm volatile("" ::: "memory");
        constexpr int RPS = 64 / CPW;          // rows per store instruction
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) {
            const int rr = i * RPS + lane / CPW;
            const int lq = lane % CPW;
            const u32x4 v = *(const u32x4 *)(wreg + rr * (CPW * 16) + ((lq ^ (rr & (CPW - 1))) * 16));
            const int mr = row0 + rtw * 32 + rr;   // the row's index among the (b, c) rows
            if (mr < rows) {
                const int nd = mr / p.G;
                const int64_t nn = R.off + nd;
                const int qr = c * p.G + (mr - nd * p.G);
                const int col = (ks + KS * (lq >> 2)) * 32 + (lq & 3) * 8;
                store_through(gmem(p.ws_o + (((int64_t)u.s * p.N + nn) * p.Hq + qr) * D) + col, v);
            }
        }
        return;
    }
    if (row_ok) {
        const auto orow = gmem(p.ws_o + (((int64_t)u.s * p.N + n) * p.Hq + qh) * D);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (!owns_dt(dt))
                continue;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f16x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (_Float16)__builtin_ldexpf(acc_o[dt][i4 * 4 + j] * inv, -ex);
                store_through(orow + dt * 32 + i4 * 8 + hh * 4, __builtin_bit_cast(u32x2, v));
            }
        }
        if (lse_writer)
            store_through(&gmem((f32x2 *)p.ws_ml)[((int64_t)u.s * p.N + n) * p.Hq + qh], __builtin_bit_cast(u32x2, f32x2{lse2, (float)ex}));
    }
}

// ---------------------------------------------------------------------------
// split-K merge: one wave per (node, q head) row, over all N * Hq rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(FwdParams p_arg)
{
    const FwdParams p = load_args(p_arg);
    const int64_t r0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // n * Hq + qh
    if (r0 >= (int64_t)p.N * p.Hq)
        return;
    const int64_t r[1] = {r0};
    const bool on[1] = {true};
    merge_rows_rb<D, 1>(p, r, on, threadIdx.x & 63);
}

// ---------------------------------------------------------------------------
// split-K merge for many rows and few splits: D / 8 lanes per row (64 * 8 / D
// rows per wave), each lane merging its own 8 output columns over every
// split, so no step crosses lanes.  Splits go in batches of BS whose partial
// slices and (lse, e) pairs are all loaded before any is used, with an online
// rescale between batches.  The same sums as merge_rows_rb (weights
// 2^{lse_s - max}, stale rows of zero-weight splits excluded by a select),
// taken in split order in each lane.
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void merge_lanes_kernel(FwdParams p_arg)
{
    constexpr int LPR = D / 8;
    constexpr int RPW = 64 / LPR;
    const FwdParams p = load_args(p_arg);
    const int64_t nrows = (int64_t)p.N * p.Hq;
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
    if (row >= nrows)
        return;   // no lane depends on another
    const int dcol = (lane % LPR) * 8;
    const int ns = p.nsplit;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, tot = 0.f;
    for (int s0 = 0; s0 < ns; s0 += BS) {
        f16x8 x[BS];
        f32x2 ml[BS];
#pragma unroll
        for (int i = 0; i < BS; ++i) {
            const int64_t rs = (int64_t)min(s0 + i, ns - 1) * nrows + row;
            ml[i] = gmem((const f32x2 *)p.ws_ml)[rs];
            x[i] = *(const __attribute__((address_space(1))) f16x8 *)(p.ws_o + rs * D + dcol);
        }
        float mb = -INFINITY;
#pragma unroll
        for (int i = 0; i < BS; ++i)
            if (s0 + i < ns)
                mb = fmaxf(mb, ml[i][0]);
        if (mb > m_run) {
            const float sc = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mb);
            tot *= sc;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] *= sc;
            m_run = mb;
        }
#pragma unroll
        for (int i = 0; i < BS; ++i) {
            if (s0 + i < ns) {
                const float l2 = ml[i][0];
                const float wgt = l2 == -INFINITY ? 0.f : fast_exp2(l2 - m_run);
                tot += wgt;
                if (wgt > 0.f) {
                    const float wo = __builtin_ldexpf(wgt, (int)ml[i][1]);   // weight of the scaled row
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[j] += wo * (float)x[i][j];
                }
            }
        }
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    u32x4 w4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 e0 = (__bf16)(acc[2 * j] * inv);
        const __bf16 e1 = (__bf16)(acc[2 * j + 1] * inv);
        w4[j] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
    }
    *(__attribute__((address_space(1))) u32x4 *)(gmem((uint16_t *)p.out) + row * D + dcol) = w4;
    if (dcol == 0)
        gmem(p.lse)[row] = tot > 0.f ? (m_run + __builtin_log2f(tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 forward: one wave per (node, q head) row, 64 keys per step.  Lanes
// take keys for the scores (each lane's K row read as 16-byte vectors, all in
// flight, four partial dot products), the softmax reductions run on DPP and
// lane swaps, the visible keys' weights and rows are compacted in LDS, and
// lanes take head-dim elements for P V with 32 / (D / 64) V rows in flight.
// No split (nsplit == 1).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p)
{
    constexpr int PER = D / 64;
    constexpr int D4 = D / 4;
    constexpr int U = 32 / PER;   // V rows in flight (32 registers of them)
    __shared__ float4 qs[4][D4];
    __shared__ float pl[4][64];
    __shared__ int64_t rl[4][64];
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
    if (live && lane < D4)
        qs[wv][lane] = ((const float4 *)p.q)[(n * p.Hq + qh) * D4 + lane];
    __syncthreads();
    if (!live)
        return;   // no barrier after this point
    const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
    const uint64_t *mrow = p.anc_mask + n * kMaskWords;
    const float *kc_base = (const float *)p.k_cache;
    const float *vc_base = (const float *)p.v_cache;
    const float *kt_base = (const float *)p.k_tree;
    const float *vt_base = (const float *)p.v_tree;
    auto fmax_op = [](float a, float x) { return fmaxf(a, x); };
    auto add_op = [](float a, float x) { return a + x; };

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
            const float4 *kr = (const float4 *)(kb + r);
            float4 kv[D4];
#pragma unroll
            for (int i = 0; i < D4; ++i)
                kv[i] = kr[i];
            float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < D4; ++i) {
                const float4 qv = qs[wv][i];
                float &a = a4[i & 3];
                a = __builtin_fmaf(qv.x, kv[i].x, a);
                a = __builtin_fmaf(qv.y, kv[i].y, a);
                a = __builtin_fmaf(qv.z, kv[i].z, a);
                a = __builtin_fmaf(qv.w, kv[i].w, a);
            }
            s = ((a4[0] + a4[1]) + (a4[2] + a4[3])) * p.c2;
        }
        const float mx = wave_reduce(s, fmax_op);
        const float m_new = fmaxf(m_run, mx);
        if (m_new == -INFINITY)
            continue;   // nothing visible yet in this chunk or before
        const float alpha = fast_exp2(m_run - m_new);
        const float pv = (r >= 0) ? fast_exp2(s - m_new) : 0.f;
        l_run = l_run * alpha + wave_reduce(pv, add_op);
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc[e] *= alpha;
        // the visible keys of this step, compacted in lane order
        const uint64_t vis = __ballot(r >= 0);
        const int nvis = __builtin_popcountll(vis);
        if (r >= 0) {
            const int idx = __builtin_popcountll(vis & ((1ull << lane) - 1ull));
            pl[wv][idx] = pv;
            rl[wv][idx] = r;
        }
        for (int j0 = 0; j0 < nvis; j0 += U) {
            float pj[U];
            float v[U][PER];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int jj = min(j0 + u, nvis - 1);   // past the end: a visible row, weight 0
                pj[u] = j0 + u < nvis ? pl[wv][jj] : 0.f;
                const float *vr = vb + rl[wv][jj];
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    v[u][e] = vr[lane + 64 * e];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    acc[e] = __builtin_fmaf(pj[u], v[u][e], acc[e]);
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
template <int D, int NR, int KS, int NSTG = 2>
static void launch_fwd_bf16_t(const FwdParams &p, hipStream_t stream)
{
    const dim3 grid(p.units_per_xcd * 8), block(NR * KS * 64);
    if (p.page_shift >= 4)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NR, KS, true, NSTG>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NR, KS, false, NSTG>), grid, block, 0, stream, p);
}

hipError_t launch_fwd(const FwdParams &p, int dtype_fp32, int nr, int ks, int nstg, hipStream_t stream)
{
    if (dtype_fp32) {
        const dim3 row_grid((p.max_tree * p.Hq + 3) / 4, p.B);
        if (p.D == 64)
            hipLaunchKernelGGL((fwd_f32_kernel<64>), row_grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_f32_kernel<128>), row_grid, dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    // (row tiles, key slices, stages) chosen by the host; anything else is a
    // host bug and fails the launch
    if (nstg != 2 && !(nstg == 4 && p.D == 128 && nr == 8 && ks == 1))
        return hipErrorInvalidValue;
    if (p.D == 64) {
        if (nr == 1 && ks == 2) launch_fwd_bf16_t<64, 1, 2>(p, stream);
        else if (nr == 2 && ks == 2) launch_fwd_bf16_t<64, 2, 2>(p, stream);
        else if (nr == 4 && ks == 2) launch_fwd_bf16_t<64, 4, 2>(p, stream);
        else if (nr == 8 && ks == 1) launch_fwd_bf16_t<64, 8, 1>(p, stream);
        else return hipErrorInvalidValue;
    } else {
        if (nr == 1 && ks == 4) launch_fwd_bf16_t<128, 1, 4>(p, stream);
        else if (nr == 2 && ks == 2) launch_fwd_bf16_t<128, 2, 2>(p, stream);
        else if (nr == 4 && ks == 2) launch_fwd_bf16_t<128, 4, 2>(p, stream);
        else if (nr == 4 && ks == 1) launch_fwd_bf16_t<128, 4, 1>(p, stream);
        else if (nr == 8 && ks == 1 && nstg == 4) launch_fwd_bf16_t<128, 8, 1, 4>(p, stream);
        else if (nr == 8 && ks == 1) launch_fwd_bf16_t<128, 8, 1>(p, stream);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const FwdParams &p, hipStream_t stream)
{
    if (p.nsplit == 1)
        return hipSuccess;
    const int64_t nrows = (int64_t)p.N * p.Hq;
    if (nrows >= kMergeLanesMinRows && p.nsplit <= 16) {
        // many rows, few splits: lanes per row (budget-256 and mixed batches:
        // 5.2 -> 3.7 and 8.3 -> 4.8 us); with few rows one wave per row keeps
        // more loads in flight (512 rows, 17 splits: 2.9 against 4.3 us)
        const int rpw = 64 / (p.D / 8);
        const dim3 grid((unsigned)((nrows + 4 * rpw - 1) / (4 * rpw)));
#define TA_MERGE_LANES(DV, BSV) hipLaunchKernelGGL((merge_lanes_kernel<DV, BSV>), grid, dim3(256), 0, stream, p)
        if (p.D == 64) {
            if (p.nsplit <= 8)
                TA_MERGE_LANES(64, 8);
            else
                TA_MERGE_LANES(64, 16);
        } else {
            if (p.nsplit <= 8)
                TA_MERGE_LANES(128, 8);
            else
                TA_MERGE_LANES(128, 16);
        }
#undef TA_MERGE_LANES
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((nrows + 3) / 4));
    if (p.D == 64)
        hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ta
