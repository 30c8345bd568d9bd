// Internal interface between the host dispatch (tree_attn.cpp) and the
// device code (attn.hip, plan.hip, tree.hip, commit.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta {

constexpr int kMaskWords = 4;
constexpr int kMaxTree = 64 * kMaskWords;
constexpr int kTreeOk = 0;
constexpr int kTreeBadOffsets = -1;
constexpr int kTreeBadPrefix = -2;
constexpr int kBlockKeys = 64;   // keys per LDS block of the forward kernel
constexpr int kMaxSplits = 64;   // merge uses one lane per split
constexpr int64_t kMergeLanesMinRows = 4096;   // merge: lanes per row from here on

struct PlanParams {
    const int32_t *parent;
    const int32_t *tree_off;
    const int32_t *prefix_len;
    uint64_t *anc_mask;
    int32_t *depth;
    int32_t *pos_id;
    int32_t *status;
    int32_t B, N, max_tree;
};

// depth-first relabelling: the plan's inputs and outputs (written in the new
// labelling) plus the permutation, its inverse and the relabelled parents
struct PlanDfsParams {
    const int32_t *parent;
    const int32_t *tree_off;
    const int32_t *prefix_len;
    int32_t *perm;          // [N] new global index -> old global index
    int32_t *inv_perm;      // [N] old -> new
    int32_t *parent_new;    // [N] local parents in the new labelling
    uint64_t *anc_mask;
    int32_t *depth;
    int32_t *pos_id;
    int32_t *status;
    int32_t B, N, max_tree;
};

struct GatherParams {
    const void *src;
    const int32_t *index;
    void *dst;
    int64_t n_src, n_rows, row_bytes;
};

struct FwdParams {
    const void *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len, *tree_off;
    const uint64_t *anc_mask;
    void *out;
    float *lse;
    // split-K workspace (nsplit > 1):
    uint16_t *ws_o;    // [nsplit, N, Hq, D] normalised partial outputs, each row
                       // scaled by 2^-e into fp16 range (fp16 bit patterns)
    float *ws_ml;      // [nsplit, N, Hq, 2] (partial log2-sum-exp of the scaled
                       // scores, e) per partial row
    int32_t B, N, Hq, Hkv, G, D;
    int32_t num_pages, max_pages, page_shift, max_tree;
    int32_t nsplit, chunk;          // split slots and prefix keys per slot
    int32_t tree_slot;              // 1: with nsplit > 1 the last slot runs the
                                    // tree alone; 0: a request's tree rides with
                                    // its last non-empty prefix chunk
    int32_t n_rt;                   // row tiles per (request, kv head)
    int32_t units, units_per_xcd;   // work units and their per-XCD share
    float c2;                       // softmax scale * log2(e)
    // Plan built inside the attention kernel (bf16 only): with parent set,
    // the workgroups that own a request's tree derive the ancestor masks from
    // the parent array instead of reading anc_mask, and write the plan's
    // outputs (all four are then set; null otherwise).
    const int32_t *parent;
    uint64_t *plan_mask;
    int32_t *plan_depth, *plan_pos, *plan_status;
};

struct CommitParams {
    const uint64_t *anc_mask;
    const int32_t *depth, *tree_off, *prefix_len, *accepted, *block_table;
    const char *k_tree, *v_tree;
    char *k_cache, *v_cache;
    int32_t *new_prefix_len, *status;
    int32_t B, N, row_bytes, page_shift, num_pages, max_pages, max_tree;
};

constexpr int kCommitBadAccepted = -3;
constexpr int kCommitBadPage = -4;
constexpr int kCommitBadPlan = -5;

struct TreeParams {
    const float *logp;   // [B, Dmax, K]
    int32_t *parent, *choice;
    float *score;        // [B, T] each
    int32_t B, Dmax, K, T;
};
constexpr int kTreeMaxK = 64;          // candidates per depth (one lane each)
constexpr int kTreeMaxDepth = 64;
constexpr int kTreeMaxPool = 16448;    // K * (T + 1) candidate slots
constexpr int kTreeMaxLogp = 4096;     // Dmax * K

hipError_t launch_plan(const PlanParams &p, hipStream_t stream);
hipError_t launch_plan_dfs(const PlanDfsParams &p, hipStream_t stream);
hipError_t launch_gather(const GatherParams &p, hipStream_t stream);
// best-first draft trees: one workgroup per request
hipError_t launch_build_tree(const TreeParams &p, hipStream_t stream);
// accepted-path commit: one workgroup per request
hipError_t launch_commit(const CommitParams &p, hipStream_t stream);
// nr: 32-row tiles per workgroup of the bf16 kernel; ks: waves per row tile
// that split each step's keys; nstg: K/V stages in LDS, 2, or 4 for 8 row
// tiles with one slice at head_dim 128 (see fwd_bf16_kernel)
hipError_t launch_fwd(const FwdParams &p, int dtype_fp32, int nr, int ks, int nstg, hipStream_t stream);
// split-K merge of the partials written by launch_fwd (no-op for one split)
hipError_t launch_merge(const FwdParams &p, hipStream_t stream);

}  // namespace ta
