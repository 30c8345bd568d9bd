// Host side of the C ABI declared in include/tree_attn.h: argument checks,
// the split-K choice, workspace layout and kernel dispatch.  Every check runs
// before any HIP call so that bad arguments never reach the device.
#include <algorithm>
#include <initializer_list>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"
#include "tree_attn.h"

namespace {

// MI355X has 256 CUs; the bf16 kernel runs 2 waves per SIMD, i.e. 8 waves
// (8 / NW workgroups) per CU.  Splits are added until the grid fills that.
constexpr int64_t kNumCUs = 256;
constexpr int64_t kWavesPerCU = 8;
// (request, kv head, 128-row tile) units from which 4-wave workgroups pay
constexpr int64_t kWideUnits = 128;
// prefix length from which the 8-wave workgroups' units are long enough for
// copies issued three steps ahead (four K/V stages) to pay
constexpr int64_t kDeepPrefix = 1024;
// longest prefix chunk, in keys, that a single request's 8-wave units are
// given while the GPU has CUs to spare
constexpr int64_t kLongChunk = 640;
// prefix length from which a single request's tree rides with its last prefix
// chunk instead of taking a slot of its own
constexpr int64_t kTreeRidesPrefix = 4096;

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t ilog2(int32_t x)
{
    int32_t r = 0;
    while ((1 << r) < x)
        ++r;
    return r;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

#ifndef TA_MAX_WAVES
#define TA_MAX_WAVES 8
#endif

// waves per workgroup of the bf16 kernel: enough 32-row tiles for the rows
// of one (request, kv head), at most TA_MAX_WAVES (up to 256 rows share each
// K/V block in LDS)
int32_t waves_for(int32_t rows)
{
    if (rows <= 32)
        return 1;
    if (rows <= 64 || TA_MAX_WAVES == 2)
        return 2;
    if (rows <= 128 || TA_MAX_WAVES == 4)
        return 4;
    return 8;
}

struct Geometry {
    int32_t nr, ks, n_rt, nsplit, chunk;
    int32_t nstg = 2;   // K/V stages in LDS (4: copies three steps ahead)
    bool tree_slot;     // nsplit > 1: the last slot runs the tree alone
};

// key slices per row tile (waves of one row tile that split each step's
// keys): fill the workgroup up to 8 waves; head_dim 64 has two output d
// tiles, so at most two slices
int32_t slices_for(int32_t nr, int32_t D)
{
    if (nr >= 8)
        return 1;
    // two row tiles at head_dim 128 (budget 16): two slices, i.e. 4-wave
    // workgroups, whose slice combine is half as long as with four
    // (measured on the budget-16 layer: attention kernel 11.2 -> 10.0 us)
    if (D == 64 || nr == 4 || (nr == 2 && D == 128))
        return 2;
    return 4;
}

bool sizes_ok(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_tree, int32_t max_prefix,
              ta_dtype_t dtype)
{
    return B >= 0 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && (D == 64 || D == 128) &&
           max_tree >= 0 && max_tree <= TREE_ATTN_MAX_TREE && max_prefix >= 0 &&
           (dtype == TA_DTYPE_BF16 || dtype == TA_DTYPE_FP32);
}

// Work decomposition: row tiles per (request, kv head) and split slots.
// The prefix is cut into equal chunks of whole 64-key blocks, one fewer than
// the slot target.  For a single request the last slot runs the tree phase
// alone, beside the prefix chunks.  With several requests that slot is
// dropped and each request's tree rides with its last, partial prefix chunk
// (8 requests of up to 4051 keys, budget 64: 5 chunks and no tree slot,
// attention kernel 39.9 us, against 42.4 us with a tree slot per request).
// Slots are added only while the grid is short of one full wave of the GPU,
// and are re-counted after rounding the chunk to whole blocks so that no
// trailing prefix slot is empty for the longest prefix.
Geometry geometry(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_tree,
                  int32_t max_prefix, ta_dtype_t dtype, int32_t forced_splits)
{
    Geometry g;
    const int32_t G = Hq / Hkv;
    const int32_t rows = max_tree * G;
    g.nr = waves_for(rows);
    g.ks = slices_for(g.nr, D);
    // Head_dim 128 with many rows per (request, kv head):
    // - when the 8-wave workgroups (256 rows) alone fill the GPU and walk long
    //   prefixes, they stay, with four K/V stages: copies go out three steps
    //   ahead (32 requests, budget 256, 4096-token prefixes: attention kernel
    //   579 -> 563 us; with 5-block units, as for a single request of budget
    //   256, the deeper prologue costs 2 %, so shorter prefixes keep two);
    // - else, with plenty of work units, 4-wave workgroups (4 row tiles, one
    //   slice): two fit on a CU, and as independent workgroups (no shared
    //   barrier) one's softmax overlaps the other's MFMAs (measured against
    //   8-wave ones with two stages: budget-256 and mixed batches 3-5 %
    //   faster; a single request, with few units, is not).
    if (D == 128 && g.nr == 8) {
        if ((int64_t)B * Hkv * ceil_div(rows, 256) >= kNumCUs && max_prefix >= kDeepPrefix &&
            dtype == TA_DTYPE_BF16) {
            g.nstg = 4;
        } else if ((int64_t)B * Hkv * ceil_div(rows, 128) >= kWideUnits) {
            g.nr = 4;
            g.ks = 1;
        }
    }
    g.n_rt = rows > 0 ? (int32_t)ceil_div(rows, 32 * g.nr) : 1;
    const int32_t nw = g.nr * g.ks;
    // a step of the kernel covers this many prefix keys
    const int64_t step_keys = (int64_t)ta::kBlockKeys * (g.ks == 4 ? 2 : 1);
    int64_t nslot = 1;
    if (dtype == TA_DTYPE_BF16 && max_prefix > 0) {
        if (forced_splits > 0) {
            nslot = forced_splits;
        } else {
            const int64_t base = (int64_t)B * Hkv * g.n_rt;
            // one workgroup per CU for the 4-wave budget-16 shape: more,
            // smaller prefix chunks cost more in the merge than they gain
            // (17 slots against 33 at chain16: 12.5 against 15.5 us a step)
            int64_t target = (g.nr == 2 && D == 128) ? kNumCUs : kNumCUs * (kWavesPerCU / nw);
            // With several requests the prefixes can differ in length, and
            // chunks are cut to the longest: finer chunks keep the long
            // requests' units from trailing the rest (8 requests of 512 to
            // 4051 keys, budget 64: 5 prefix chunks, attention kernel 39.9 us,
            // against 3 chunks 52.5 us and 7 chunks 46.3 us); batches of the
            // 4-wave budget-16 shape take twice the target (one-call step,
            // against 1.5 times: 16 requests 42.7 -> 40.0 us, 8 requests of
            // 2048 keys 21.2 -> 19.9 us, 12 requests 33.8 -> 27.9 us; over
            // ten such batch shapes the count is within 3 % of the best
            // forced count on eight)
            if (B > 1)
                target = (g.nr == 2 && D == 128) ? target * 2 : target * 3 / 2;
            if (base > 0 && base < target)
                nslot = ceil_div(target, base);
            if (B <= 1 && g.nr == 8 && D == 128 && base > 0) {
                // A single request with 8-wave units: each slot beyond the
                // first costs partial writes and merge reads, so the slots
                // fill three quarters of the CUs, and long prefixes take
                // more, up to one workgroup per CU, to keep chunks at most
                // kLongChunk keys.
                const int64_t lo = ceil_div(kNumCUs * 3 / 4, base);
                const int64_t hi = std::min<int64_t>(ceil_div(kNumCUs, base), 1 + ceil_div(max_prefix, kLongChunk));
                nslot = std::max<int64_t>(1, std::max(lo, hi));
            }
        }
        if (nslot > ta::kMaxSplits)
            nslot = ta::kMaxSplits;
    }
    g.chunk = (int32_t)(ceil_div(max_prefix > 0 ? max_prefix : 1, step_keys) * step_keys);
    g.nsplit = 1;
    g.tree_slot = B <= 1;
    if (nslot > 1) {
        // prefix chunks: one fewer than the slots, except that a forced count
        // without a tree slot is all prefix chunks
        int64_t npre = (forced_splits > 0 && !g.tree_slot) ? nslot : nslot - 1;
        const int64_t max_blocks = ceil_div(max_prefix, ta::kBlockKeys);
        if (npre > max_blocks)
            npre = max_blocks;
        // whole steps per chunk where the prefix allows it, whole blocks else
        const int64_t per = ceil_div(max_prefix, npre);
        const int64_t unit = per >= step_keys ? step_keys : ta::kBlockKeys;
        int64_t chunk = ceil_div(per, unit) * unit;
        npre = ceil_div(max_prefix, chunk);
        g.nsplit = (int32_t)(g.tree_slot ? npre + 1 : npre);
        g.chunk = (int32_t)chunk;
        if (g.tree_slot && forced_splits <= 0 && g.nr == 8 && step_keys == ta::kBlockKeys &&
            max_prefix >= kTreeRidesPrefix) {
            // A single request with a long prefix: the tree rides with the
            // last prefix chunk, and the chunks are cut so that this one's
            // prefix blocks plus the tree's match the others.  Graph replay,
            // budget 200-256 trees: 4096-token prefix 30.1 -> 29.6 us, 6000
            // 37.2 -> 35.8 us, 8192 46.2 -> 44.8 us.  Shorter prefixes keep
            // the tree slot: the tree phase (masks, and the plan when it is
            // built in the same call) costs more than its block count, and
            // riding lost 1-28 % there (2048: 24.2 -> 24.7 us).
            const int64_t pb = ceil_div(max_prefix, ta::kBlockKeys);
            const int64_t tb = ceil_div(max_tree, ta::kBlockKeys);
            const int64_t cb = std::max<int64_t>(1, ceil_div(pb + tb, g.nsplit));
            g.tree_slot = false;
            g.chunk = (int32_t)(cb * ta::kBlockKeys);
            g.nsplit = (int32_t)ceil_div(max_prefix, (int64_t)g.chunk);
        }
    }
    return g;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split workspace layout (nsplit > 1): the partial outputs (fp16, each row
// scaled by a power of two), then the (lse, exponent) pairs.
size_t ws_o_bytes(int32_t nsplit, int32_t N, int32_t Hq, int32_t D)
{
    return align256((size_t)nsplit * N * Hq * D * sizeof(uint16_t));
}

size_t ws_ml_bytes(int32_t nsplit, int32_t N, int32_t Hq)
{
    return align256((size_t)nsplit * N * Hq * 2 * sizeof(float));
}

size_t ws_bytes(const Geometry &g, int32_t N, int32_t Hq, int32_t D)
{
    if (g.nsplit <= 1 || N == 0)
        return 0;
    return ws_o_bytes(g.nsplit, N, Hq, D) + ws_ml_bytes(g.nsplit, N, Hq);
}

ta_status_t check_fwd(const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                      const void *v_cache, const int32_t *block_table, const int32_t *prefix_len,
                      const int32_t *tree_off, const uint64_t *anc_mask, int32_t B, int32_t N,
                      int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                      int32_t max_pages, int32_t max_tree, int32_t max_prefix, float scale,
                      ta_dtype_t dtype, int32_t num_splits, const void *out, const float *lse,
                      const void *workspace, size_t workspace_bytes)
{
    if (dtype != TA_DTYPE_BF16 && dtype != TA_DTYPE_FP32)
        return TA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128)
        return TA_ERR_UNSUPPORTED;
    if (max_tree > TREE_ATTN_MAX_TREE)
        return TA_ERR_UNSUPPORTED;
    if (page_size < 1 || page_size > 1024 || !is_pow2(page_size))
        return TA_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_tree < 0 || max_prefix < 0 ||
        num_pages < 0 || max_pages < 0 || num_splits < 0 || num_splits > ta::kMaxSplits)
        return TA_ERR_BAD_SHAPE;
    if ((int64_t)N > (int64_t)B * max_tree || B > 65535)
        return TA_ERR_BAD_SHAPE;
    if ((int64_t)max_prefix > (int64_t)max_pages * page_size)
        return TA_ERR_BAD_SHAPE;
    if (max_prefix > 0 && num_pages < 1)
        return TA_ERR_BAD_SHAPE;
    // element counts must fit the kernels' 64-bit offsets with room to spare,
    // and per-row index math uses 32-bit node and head ids
    if ((int64_t)N * Hq > INT32_MAX || (int64_t)B * max_pages > INT32_MAX ||
        (int64_t)num_pages * page_size * Hkv * D > ((int64_t)1 << 46))
        return TA_ERR_BAD_SHAPE;
    if (!(scale == scale) || isinf(scale))
        return TA_ERR_BAD_SHAPE;
    if (B == 0 || N == 0)
        return TA_OK;
    if (!q || !k_tree || !v_tree || !prefix_len || !tree_off || !anc_mask || !out || !lse)
        return TA_ERR_NULL_PTR;
    if (max_prefix > 0 && (!k_cache || !v_cache || !block_table))
        return TA_ERR_NULL_PTR;
    // the kernels move rows of q, k, v and out as 16-byte vectors, mask words
    // as u64 and the rest as 32-bit words
    for (const void *ptr : {q, k_tree, v_tree, k_cache, v_cache, out})
        if (((uintptr_t)ptr & 15) != 0)
            return TA_ERR_BAD_SHAPE;
    if (((uintptr_t)anc_mask & 7) != 0 || ((uintptr_t)lse & 3) != 0 || ((uintptr_t)block_table & 3) != 0 ||
        ((uintptr_t)prefix_len & 3) != 0 || ((uintptr_t)tree_off & 3) != 0)
        return TA_ERR_BAD_SHAPE;
    const Geometry g = geometry(B, Hq, Hkv, D, max_tree, max_prefix, dtype, num_splits);
    const size_t need = ws_bytes(g, N, Hq, D);
    if (need > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
            return TA_ERR_WORKSPACE;
    }
    return TA_OK;
}

}  // namespace

extern "C" {

int tree_attn_abi_version(void) { return TREE_ATTN_ABI_VERSION; }

const char *tree_attn_status_str(int status)
{
    switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_NULL_PTR: return "a required pointer is NULL";
    case TA_ERR_BAD_SHAPE: return "inconsistent or out-of-range sizes";
    case TA_ERR_UNSUPPORTED: return "unsupported configuration (dtype, head_dim, page_size or tree size)";
    case TA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TA_ERR_HIP: return "HIP launch failed";
    case TA_ERR_SCRATCH_LIMIT: return "the call needs more split workspace than the no-allocation entry point holds";
    default: return "unknown status";
    }
}

ta_status_t tree_attn_plan(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                           int32_t B, int32_t N, int32_t max_tree, uint64_t *anc_mask, int32_t *depth,
                           int32_t *pos_id, int32_t *status, void *stream)
{
    if (max_tree > TREE_ATTN_MAX_TREE)
        return TA_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || max_tree < 0 || (int64_t)N > (int64_t)B * max_tree)
        return TA_ERR_BAD_SHAPE;
    if (B == 0)
        return TA_OK;
    if (!tree_off || !prefix_len || !status)
        return TA_ERR_NULL_PTR;
    if (N > 0 && (!parent || !anc_mask || !depth || !pos_id))
        return TA_ERR_NULL_PTR;
    ta::PlanParams p;
    p.parent = parent;
    p.tree_off = tree_off;
    p.prefix_len = prefix_len;
    p.anc_mask = anc_mask;
    p.depth = depth;
    p.pos_id = pos_id;
    p.status = status;
    p.B = B;
    p.N = N;
    p.max_tree = max_tree;
    return ta::launch_plan(p, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

ta_status_t tree_attn_plan_dfs(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                               int32_t B, int32_t N, int32_t max_tree, int32_t *perm, int32_t *inv_perm,
                               int32_t *parent_new, uint64_t *anc_mask, int32_t *depth, int32_t *pos_id,
                               int32_t *status, void *stream)
{
    if (max_tree > TREE_ATTN_MAX_TREE)
        return TA_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || max_tree < 0 || (int64_t)N > (int64_t)B * max_tree)
        return TA_ERR_BAD_SHAPE;
    if (B == 0)
        return TA_OK;
    if (!tree_off || !prefix_len || !status)
        return TA_ERR_NULL_PTR;
    if (N > 0 && (!parent || !perm || !inv_perm || !parent_new || !anc_mask || !depth || !pos_id))
        return TA_ERR_NULL_PTR;
    ta::PlanDfsParams p;
    p.parent = parent;
    p.tree_off = tree_off;
    p.prefix_len = prefix_len;
    p.perm = perm;
    p.inv_perm = inv_perm;
    p.parent_new = parent_new;
    p.anc_mask = anc_mask;
    p.depth = depth;
    p.pos_id = pos_id;
    p.status = status;
    p.B = B;
    p.N = N;
    p.max_tree = max_tree;
    return ta::launch_plan_dfs(p, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

ta_status_t tree_attn_gather_rows(const void *src, int64_t n_src, const int32_t *index, void *dst,
                                  int64_t n_rows, int64_t row_bytes, void *stream)
{
    if (n_src < 0 || n_rows < 0 || row_bytes < 0 || row_bytes % 4 != 0 || n_src > INT32_MAX)
        return TA_ERR_BAD_SHAPE;
    if (n_rows == 0 || row_bytes == 0)
        return TA_OK;
    if (!index || !dst || (n_src > 0 && !src))
        return TA_ERR_NULL_PTR;
    if (((uintptr_t)src | (uintptr_t)dst) % 4 != 0)
        return TA_ERR_UNSUPPORTED;
    ta::GatherParams p;
    p.src = src;
    p.index = index;
    p.dst = dst;
    p.n_src = n_src;
    p.n_rows = n_rows;
    p.row_bytes = row_bytes;
    return ta::launch_gather(p, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

ta_status_t tree_attn_build_tree(const float *logp, int32_t B, int32_t max_depth, int32_t K,
                                 int32_t T, int32_t *parent, int32_t *choice, float *score,
                                 void *stream)
{
    if (K > ta::kTreeMaxK || max_depth > ta::kTreeMaxDepth || T > TREE_ATTN_MAX_TREE)
        return TA_ERR_UNSUPPORTED;
    if (B < 0 || K < 1 || max_depth < 1 || T < 0)
        return TA_ERR_BAD_SHAPE;
    if ((int64_t)K * (T + 1) > ta::kTreeMaxPool || (int64_t)K * max_depth > ta::kTreeMaxLogp)
        return TA_ERR_UNSUPPORTED;
    // the implicit tree (K children per node, max_depth levels) must hold T nodes
    double nodes = 0, level = 1;
    for (int32_t d = 0; d < max_depth && nodes < T; ++d) {
        level *= K;
        nodes += level;
    }
    if (nodes < T)
        return TA_ERR_BAD_SHAPE;
    if (B == 0 || T == 0)
        return TA_OK;
    if (!logp || !parent || !choice || !score)
        return TA_ERR_NULL_PTR;
    ta::TreeParams p;
    p.logp = logp;
    p.parent = parent;
    p.choice = choice;
    p.score = score;
    p.B = B;
    p.Dmax = max_depth;
    p.K = K;
    p.T = T;
    return ta::launch_build_tree(p, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

ta_status_t tree_attn_commit(const uint64_t *anc_mask, const int32_t *depth, const int32_t *tree_off,
                             const int32_t *prefix_len, const int32_t *accepted, const void *k_tree,
                             const void *v_tree, void *k_cache, void *v_cache,
                             const int32_t *block_table, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                             int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq,
                             int32_t max_tree, ta_dtype_t dtype, int32_t *new_prefix_len,
                             int32_t *status, void *stream)
{
    if (dtype != TA_DTYPE_BF16 && dtype != TA_DTYPE_FP32)
        return TA_ERR_UNSUPPORTED;
    if (max_tree > TREE_ATTN_MAX_TREE || page_size < 1 || page_size > 1024 ||
        (page_size & (page_size - 1)) != 0)
        return TA_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || Hkv < 1 || D < 1 || max_tree < 0 || num_pages < 0 ||
        max_pages_per_seq < 0 || (int64_t)N > (int64_t)B * max_tree)
        return TA_ERR_BAD_SHAPE;
    const int64_t row_bytes = (int64_t)Hkv * D * (dtype == TA_DTYPE_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || row_bytes > INT32_MAX)
        return TA_ERR_UNSUPPORTED;
    if (B == 0)
        return TA_OK;
    if (!tree_off || !prefix_len || !accepted || !new_prefix_len || !status || !block_table ||
        !k_cache || !v_cache)
        return TA_ERR_NULL_PTR;
    if (N > 0 && (!anc_mask || !depth || !k_tree || !v_tree))
        return TA_ERR_NULL_PTR;
    // rows are copied 16 bytes at a time
    for (const void *ptr : {k_tree, v_tree, (const void *)k_cache, (const void *)v_cache})
        if (ptr && ((uintptr_t)ptr & 15) != 0)
            return TA_ERR_BAD_SHAPE;
    ta::CommitParams p;
    p.anc_mask = anc_mask;
    p.depth = depth;
    p.tree_off = tree_off;
    p.prefix_len = prefix_len;
    p.accepted = accepted;
    p.block_table = block_table;
    p.k_tree = (const char *)k_tree;
    p.v_tree = (const char *)v_tree;
    p.k_cache = (char *)k_cache;
    p.v_cache = (char *)v_cache;
    p.new_prefix_len = new_prefix_len;
    p.status = status;
    p.B = B;
    p.N = N;
    p.row_bytes = (int32_t)row_bytes;
    p.page_shift = ilog2(page_size);
    p.num_pages = num_pages;
    p.max_pages = max_pages_per_seq;
    p.max_tree = max_tree;
    return ta::launch_commit(p, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

int32_t tree_attn_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_tree,
                             int32_t max_prefix, ta_dtype_t dtype)
{
    if (!sizes_ok(B, Hq, Hkv, D, max_tree, max_prefix, dtype))
        return 0;
    return geometry(B, Hq, Hkv, D, max_tree, max_prefix, dtype, 0).nsplit;
}

size_t tree_attn_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_tree, int32_t max_prefix, ta_dtype_t dtype,
                                 int32_t num_splits)
{
    if (!sizes_ok(B, Hq, Hkv, D, max_tree, max_prefix, dtype) || N < 0 || num_splits < 0 ||
        num_splits > ta::kMaxSplits)
        return 0;
    return ws_bytes(geometry(B, Hq, Hkv, D, max_tree, max_prefix, dtype, num_splits), N, Hq, D);
}

ta_status_t tree_attn_fwd_check(const void *q, const void *k_tree, const void *v_tree,
                                const void *k_cache, const void *v_cache, const int32_t *block_table,
                                const int32_t *prefix_len, const int32_t *tree_off,
                                const uint64_t *anc_mask, int32_t B, int32_t N, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                int32_t max_pages_per_seq, int32_t max_tree, int32_t max_prefix,
                                float softmax_scale, ta_dtype_t dtype, int32_t num_splits,
                                const void *out, const float *lse, const void *workspace,
                                size_t workspace_bytes)
{
    return check_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask,
                     B, N, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq, max_tree, max_prefix,
                     softmax_scale, dtype, num_splits, out, lse, workspace, workspace_bytes);
}

}  // extern "C"

namespace {

enum Stage { kStagePartial = 1, kStageMerge = 2, kStageBoth = 3 };

// the plan's inputs and outputs when the attention kernel builds the plan
struct FusedPlan {
    const int32_t *parent;
    uint64_t *anc_mask;
    int32_t *depth, *pos_id, *status;
};

ta_status_t run_fwd(const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                    const void *v_cache, const int32_t *block_table, const int32_t *prefix_len,
                    const int32_t *tree_off, const uint64_t *anc_mask, int32_t B, int32_t N,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                    int32_t max_pages_per_seq, int32_t max_tree, int32_t max_prefix,
                    float softmax_scale, ta_dtype_t dtype, int32_t num_splits, void *out, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream, int stages,
                    const FusedPlan *fp = nullptr)
{
    const ta_status_t st = check_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                                     tree_off, anc_mask, B, N, Hq, Hkv, D, page_size, num_pages,
                                     max_pages_per_seq, max_tree, max_prefix, softmax_scale, dtype,
                                     num_splits, out, lse, workspace, workspace_bytes);
    if (st != TA_OK || B == 0 || N == 0)
        return st;
    const Geometry g = geometry(B, Hq, Hkv, D, max_tree, max_prefix, dtype, num_splits);
    const int64_t units = (int64_t)B * Hkv * g.nsplit * g.n_rt;
    if (units > INT32_MAX - 8)
        return TA_ERR_BAD_SHAPE;
    ta::FwdParams p;
    p.q = q;
    p.k_tree = k_tree;
    p.v_tree = v_tree;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.prefix_len = prefix_len;
    p.tree_off = tree_off;
    p.anc_mask = anc_mask;
    p.out = out;
    p.lse = lse;
    p.ws_o = nullptr;
    p.ws_ml = nullptr;
    if (g.nsplit > 1) {
        p.ws_o = (uint16_t *)workspace;
        p.ws_ml = (float *)((char *)workspace + ws_o_bytes(g.nsplit, N, Hq, D));
    }
    p.B = B;
    p.N = N;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.D = D;
    p.num_pages = num_pages;
    // without a prefix the block table may be null: no page is ever read
    p.max_pages = max_prefix > 0 ? max_pages_per_seq : 0;
    p.page_shift = ilog2(page_size);
    p.max_tree = max_tree;
    p.nsplit = g.nsplit;
    p.chunk = g.chunk;
    p.tree_slot = g.tree_slot ? 1 : 0;
    p.n_rt = g.n_rt;
    p.units = (int32_t)units;
    p.units_per_xcd = (int32_t)ceil_div(units, 8);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    p.c2 = scale * 1.44269504088896340736f;
    p.parent = fp ? fp->parent : nullptr;
    p.plan_mask = fp ? fp->anc_mask : nullptr;
    p.plan_depth = fp ? fp->depth : nullptr;
    p.plan_pos = fp ? fp->pos_id : nullptr;
    p.plan_status = fp ? fp->status : nullptr;
    hipStream_t s = (hipStream_t)stream;
    if (stages & kStagePartial) {
        if (ta::launch_fwd(p, dtype == TA_DTYPE_FP32, g.nr, g.ks, g.nstg, s) != hipSuccess)
            return TA_ERR_HIP;
    }
    if (stages & kStageMerge) {
        if (ta::launch_merge(p, s) != hipSuccess)
            return TA_ERR_HIP;
    }
    return TA_OK;
}

}  // namespace

#define TA_FWD_PARAMS                                                                               \
    const void *q, const void *k_tree, const void *v_tree, const void *k_cache, const void *v_cache, \
        const int32_t *block_table, const int32_t *prefix_len, const int32_t *tree_off,              \
        const uint64_t *anc_mask, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,          \
        int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq, int32_t max_tree,           \
        int32_t max_prefix, float softmax_scale, ta_dtype_t dtype, int32_t num_splits, void *out,    \
        float *lse, void *workspace, size_t workspace_bytes, void *stream
#define TA_FWD_ARGS                                                                                 \
    q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask, B, N, Hq, Hkv, \
        D, page_size, num_pages, max_pages_per_seq, max_tree, max_prefix, softmax_scale, dtype,      \
        num_splits, out, lse, workspace, workspace_bytes, stream

extern "C" {

ta_status_t tree_attn_fwd(TA_FWD_PARAMS) { return run_fwd(TA_FWD_ARGS, kStageBoth); }

ta_status_t tree_attn_fwd_partial(TA_FWD_PARAMS) { return run_fwd(TA_FWD_ARGS, kStagePartial); }

ta_status_t tree_attn_merge(TA_FWD_PARAMS) { return run_fwd(TA_FWD_ARGS, kStageMerge); }

}  // extern "C"

namespace {

ta_status_t run_plan_fwd(const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                         const void *v_cache, const int32_t *block_table, const int32_t *prefix_len,
                         const int32_t *tree_off, const int32_t *parent, int32_t B, int32_t N, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                         int32_t max_pages_per_seq, int32_t max_tree, int32_t max_prefix,
                         float softmax_scale, ta_dtype_t dtype, int32_t num_splits, uint64_t *anc_mask,
                         int32_t *depth, int32_t *pos_id, int32_t *status, void *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream, int stages)
{
    const ta_status_t st = check_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                                     tree_off, anc_mask, B, N, Hq, Hkv, D, page_size, num_pages,
                                     max_pages_per_seq, max_tree, max_prefix, softmax_scale, dtype,
                                     num_splits, out, lse, workspace, workspace_bytes);
    if (st != TA_OK || B == 0)
        return st;
    // the plan's own pointer rules
    if (!tree_off || !prefix_len || !status)
        return TA_ERR_NULL_PTR;
    if (N > 0 && (!parent || !anc_mask || !depth || !pos_id))
        return TA_ERR_NULL_PTR;
    if (dtype == TA_DTYPE_FP32 || N == 0) {
        // the fp32 kernel reads the mask words: plan first, then attention
        const ta_status_t sp = tree_attn_plan(parent, tree_off, prefix_len, B, N, max_tree, anc_mask, depth,
                                              pos_id, status, stream);
        if (sp != TA_OK)
            return sp;
        return run_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask, B,
                       N, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq, max_tree, max_prefix,
                       softmax_scale, dtype, num_splits, out, lse, workspace, workspace_bytes, stream,
                       stages);
    }
    const FusedPlan fp = {parent, anc_mask, depth, pos_id, status};
    return run_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask, B, N,
                   Hq, Hkv, D, page_size, num_pages, max_pages_per_seq, max_tree, max_prefix, softmax_scale,
                   dtype, num_splits, out, lse, workspace, workspace_bytes, stream, stages, &fp);
}

}  // namespace

#define TA_PLAN_FWD_PARAMS                                                                               \
    const void *q, const void *k_tree, const void *v_tree, const void *k_cache, const void *v_cache,     \
        const int32_t *block_table, const int32_t *prefix_len, const int32_t *tree_off,                  \
        const int32_t *parent, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,                 \
        int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq, int32_t max_tree,               \
        int32_t max_prefix, float softmax_scale, ta_dtype_t dtype, int32_t num_splits,                   \
        uint64_t *anc_mask, int32_t *depth, int32_t *pos_id, int32_t *status, void *out, float *lse,     \
        void *workspace, size_t workspace_bytes, void *stream
#define TA_PLAN_FWD_ARGS                                                                                 \
    q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, parent, B, N, Hq, Hkv, D,    \
        page_size, num_pages, max_pages_per_seq, max_tree, max_prefix, softmax_scale, dtype, num_splits, \
        anc_mask, depth, pos_id, status, out, lse, workspace, workspace_bytes, stream

extern "C" {

ta_status_t tree_attn_plan_fwd(TA_PLAN_FWD_PARAMS) { return run_plan_fwd(TA_PLAN_FWD_ARGS, kStageBoth); }

ta_status_t tree_attn_plan_fwd_partial(TA_PLAN_FWD_PARAMS)
{
    return run_plan_fwd(TA_PLAN_FWD_ARGS, kStagePartial);
}

}  // extern "C"
