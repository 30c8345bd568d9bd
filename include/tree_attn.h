/*
 * tree_attn.h -- C ABI of the tree-causal paged attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (JetFlow: Breaking the Scaling Ceiling of Speculative
 * Decoding with Parallel Tree Drafting -- technical summary, section 2, core
 * architecture, "tree-causal attention mask", and the branch factorisation
 * equation in the same paragraph): every node of a drafted token tree attends
 * to the original input prefix and to its in-tree ancestors, itself included,
 * and never to its descendants or to unrelated sibling branches.  The same
 * operation serves the causal parallel draft head and target-model tree
 * verification, where the prefix lives in a paged KV cache (section 3,
 * "industrial integration": a paged FlashAttention with tree-mask staging).
 *
 * Two device entry points make up one decode step's attention:
 *   tree_attn_plan  parent array  -> ancestor bitmask, depth, position ids
 *   tree_attn_fwd   GQA attention over the paged prefix plus the tree's own
 *                   K/V under the ancestor bitmask; online softmax; fp32 LSE
 * (tree_attn_plan_fwd does both in one call, building the plan inside the
 * attention kernel)
 * and the steps next to it:
 *   tree_attn_build_tree   best-first draft trees from per-depth candidates
 *   tree_attn_commit       accepted root path -> the paged K/V cache
 *   tree_attn_plan_dfs     the plan in a depth-first relabelling, plus the
 *                          permutation (tree_attn_gather_rows moves rows)
 *
 * Conventions shared by every call:
 *  - All device buffers are allocated and owned by the caller; the library
 *    allocates nothing and keeps no state.  Calls are reentrant.
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    (host) pointers are host memory.  Every layout is row-major, contiguous.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *    work is enqueued on it and the call returns without synchronising.
 *  - Errors the host can see (null pointers, bad sizes, unsupported
 *    configurations, a short workspace) are returned synchronously before
 *    anything is launched.  TA_ERR_HIP reports a failed launch.  Outputs are
 *    undefined after any error.
 *  - Requests are numbered b = 0..B-1; request b owns tree nodes
 *    tree_off[b] .. tree_off[b+1]-1 (global node ids, cu_seqlens style).
 *    Inside a request nodes use local ids 0..T_b-1, T_b = tree_off[b+1] -
 *    tree_off[b], in topological order: parent[i] < i, and parent[i] = -1
 *    means node i hangs directly off the prefix (a forest is allowed).
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TREE_ATTN_ABI_VERSION 1
/* u64 words per node row of the ancestor bitmask (fixed, so plan and fwd can
 * never disagree on the layout); bit j of word w is local node 64*w + j. */
#define TREE_ATTN_MASK_WORDS 4
/* largest tree a request may have: 64 * TREE_ATTN_MASK_WORDS */
#define TREE_ATTN_MAX_TREE 256

typedef enum {
    TA_OK = 0,
    TA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                    */
    TA_ERR_BAD_SHAPE = 2,   /* inconsistent or out-of-range sizes            */
    TA_ERR_UNSUPPORTED = 3, /* valid but not implemented (dtype, head_dim..) */
    TA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required    */
    TA_ERR_HIP = 5,         /* a HIP launch failed                           */
    TA_ERR_SCRATCH_LIMIT = 6 /* tree_attn_fwd_noalloc: the call needs more
                                split workspace than its fixed array holds */
} ta_status_t;

typedef enum {
    TA_DTYPE_BF16 = 0, /* bf16 Q/K/V/O, fp32 accumulation, bf16 MFMA          */
    TA_DTYPE_FP32 = 1  /* fp32 Q/K/V/O, fp32 arithmetic throughout            */
} ta_dtype_t;

/* Per-request codes that tree_attn_plan writes into status[b]. */
#define TA_TREE_OK 0
#define TA_TREE_BAD_OFFSETS (-1) /* tree_off[0] != 0, tree_off[B] != N, a
                                    negative tree size, or T_b > max_tree   */
#define TA_TREE_BAD_PREFIX (-2)  /* prefix_len[b] < 0                       */
/* status[b] = k > 0: local node k-1 is the first node whose parent is not in
 * [-1, k-2] (not topologically ordered).  Codes are checked in the order
 * offsets, prefix, parents; the first failing check is reported. */

/* ABI version of the loaded library (TREE_ATTN_ABI_VERSION). */
int tree_attn_abi_version(void);

/* Static description of a ta_status_t value; never NULL. */
const char *tree_attn_status_str(int status);

/*
 * tree_attn_plan -- the ancestor sets of every tree node.
 *
 * Defined by: JetFlow technical summary, section 2 (core architecture), the
 * tree-causal attention mask -- a node sees the prefix and its in-tree
 * ancestors, never siblings or descendants -- and the branch factorisation
 * in the same paragraph, which conditions a node's token on the path up to
 * and including the node (so A(i) holds i itself).
 *
 * For local node i of request b, A(i) = {i} U A(parent[i]) with A(-1) empty:
 * the node's root path, itself included (the set of tree keys the node sees,
 * per the mask definition above).
 *   anc_mask[n, w] (device, u64 [N, TREE_ATTN_MASK_WORDS]): bit j of word w is
 *                  set iff local node 64*w + j is in A(i), n = tree_off[b]+i.
 *   depth[n]       (device, i32 [N]): |A(i)| (>= 1).
 *   pos_id[n]      (device, i32 [N]): prefix_len[b] + depth[n] - 1, the
 *                  node's position in the flat sequence prefix ++ root path
 *                  (for rotary embeddings).
 *   status[b]      (device, i32 [B]): TA_TREE_OK or a TA_TREE_* code / k > 0
 *                  as described above.  Rows of a request with a non-zero
 *                  status are left unwritten.  Read it after synchronising.
 * Inputs (device): parent [N] i32 local ids, tree_off [B+1] i32,
 * prefix_len [B] i32.  max_tree (host) bounds every T_b, 0..256.
 * B = 0 or N = 0 is a valid no-op (status is still written for every b).
 */
ta_status_t tree_attn_plan(const int32_t *parent, const int32_t *tree_off,
                           const int32_t *prefix_len, int32_t B, int32_t N,
                           int32_t max_tree, uint64_t *anc_mask, int32_t *depth,
                           int32_t *pos_id, int32_t *status, void *stream);

/*
 * Number of split slots (split-K, merged by LSE) that tree_attn_fwd uses for
 * these sizes when num_splits = 0 is passed; a pure function of its
 * arguments.  Returns 0 for invalid sizes.  With one slot a single pass covers
 * the prefix and the tree.  With S > 1 slots the slots cover the prefix in
 * equal chunks; for a single request (B = 1) slot S-1 covers the tree alone,
 * so the tree phase runs beside the prefix chunks, and with several requests
 * each request's tree goes with its last non-empty chunk.  A forced count is
 * reduced so that every prefix chunk holds at least one 64-key block of the
 * longest prefix.
 */
int32_t tree_attn_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t max_tree, int32_t max_prefix, ta_dtype_t dtype);

/*
 * Workspace bytes tree_attn_fwd needs for these sizes and this split count
 * (num_splits = 0: the automatic choice).  0 when no workspace is needed.
 * A pure function of its arguments.
 */
size_t tree_attn_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t max_tree, int32_t max_prefix,
                                 ta_dtype_t dtype, int32_t num_splits);

/*
 * tree_attn_fwd -- tree-causal attention of every (node, q-head) row.
 *
 * Defined by: JetFlow technical summary, section 2 (core architecture), the
 * tree-causal attention mask (the keys a node sees), used both by the causal
 * parallel draft head and by target-model tree verification; section 3
 * (industrial integration) for the prefix held in a paged KV cache
 * addressed through block tables, as in the pages' vLLM integration.
 *
 * Row (n, h), n = tree_off[b] + i, kv head c = h / (Hq / Hkv) (contiguous
 * GQA groups), sees
 *   the prefix:  K_t = k_cache[block_table[b, t / page_size], t % page_size, c]
 *                for 0 <= t < prefix_len[b]   (V likewise), and
 *   the tree:    K_j = k_tree[tree_off[b] + j, c] for every j in A(i)
 *                (bits of anc_mask[n]; V likewise),
 * with s = softmax_scale * <q[n,h], K>,
 *   out[n,h] = sum softmax(s) V    (in the input dtype),
 *   lse[n,h] = ln sum exp(s)       (fp32, natural log).
 *
 * Buffers (device):
 *   q           [N, Hq, D]                         dtype
 *   k_tree      [N, Hkv, D], v_tree likewise       dtype
 *   k_cache     [num_pages, page_size, Hkv, D]     dtype (separate K and V pools)
 *   v_cache     likewise
 *   block_table [B, max_pages_per_seq] i32 physical page ids; entries past
 *               ceil(prefix_len[b] / page_size) are never read
 *   prefix_len  [B] i32,  tree_off [B+1] i32
 *   anc_mask    [N, TREE_ATTN_MASK_WORDS] u64, as written by tree_attn_plan
 *   out         [N, Hq, D] dtype;  lse [N, Hq] f32
 *   workspace   tree_attn_workspace_bytes(...) bytes, 256-byte aligned, or
 *               NULL when that is 0; its contents are scratch between calls,
 *               and one call at a time may use it (calls that share one must
 *               be ordered: the same stream, or events).  With more than one
 *               split (bf16 only) it holds each split's normalised partial
 *               output in fp16 ([splits, N, Hq, D]), each row scaled by a
 *               power of two 2^-e so that its largest magnitude lies in
 *               [2^14, 2^15) -- any finite bf16 V stays in range, and the
 *               scaling changes no rounding -- and the pairs (partial
 *               log-sum-exp, e) in fp32 ([splits, N, Hq, 2]).  The split
 *               merge then runs as a second kernel on the stream.
 * Finite inputs: K and V rows of every prefix key and tree node a request
 *   holds must be finite.  Keys a row does not see are weighted by exact
 *   zeros inside 32- or 64-key tiles, so a NaN or Inf in such a row can
 *   still reach outputs (0 * Inf is NaN); storage past a request's keys
 *   (page tails, unused pages) is never read.
 * Host sizes: max_tree >= every T_b (<= 256), max_prefix >= every
 *   prefix_len[b] (<= max_pages_per_seq * page_size).  They size the launch
 *   so no call ever reads device data on the host.
 * softmax_scale <= 0 selects 1/sqrt(D).  num_splits = 0 selects
 *   tree_attn_num_splits(...); 1..64 forces a split-slot count (see there).
 * Supported: dtype bf16 or fp32; D in {64, 128}; page_size a power of two in
 *   [1, 1024]; Hq % Hkv == 0.  Anything else is TA_ERR_UNSUPPORTED or
 *   TA_ERR_BAD_SHAPE.
 * Alignment: q, k_tree, v_tree, k_cache, v_cache and out 16-byte aligned
 *   (rows move as 16-byte vectors), anc_mask 8-byte, lse, block_table,
 *   prefix_len and tree_off 4-byte; TA_ERR_BAD_SHAPE otherwise.
 * Device-side robustness: a page id outside [0, num_pages) or a prefix
 *   longer than the block table makes the kernel skip those keys rather than
 *   read outside the pool; tree sizes above max_tree are clamped.  Such inputs
 *   are caller errors and give undefined (but memory-safe) results.
 */
ta_status_t tree_attn_fwd(const void *q, const void *k_tree, const void *v_tree,
                          const void *k_cache, const void *v_cache,
                          const int32_t *block_table, const int32_t *prefix_len,
                          const int32_t *tree_off, const uint64_t *anc_mask,
                          int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t page_size, int32_t num_pages,
                          int32_t max_pages_per_seq, int32_t max_tree,
                          int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                          int32_t num_splits, void *out, float *lse, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * tree_attn_plan_fwd -- tree_attn_plan and tree_attn_fwd in one call.
 *
 * The same tree-causal attention (JetFlow technical summary, section 2,
 * tree-causal attention mask) computed from the parent array directly.  With
 * bf16 the attention workgroups that own a request's tree stage its parents,
 * check them and walk each node's root path themselves, so the plan costs
 * no launch of its own and runs beside the prefix work; they also write the
 * plan's outputs.  With fp32 (or N = 0) the call runs tree_attn_plan and
 * then tree_attn_fwd on the stream.
 *   q .. tree_off, B .. num_splits, out, lse, workspace: as tree_attn_fwd
 *            (the same workspace size).
 *   parent   [N] i32 (device): as tree_attn_plan.
 *   anc_mask, depth, pos_id, status (device, written): exactly what
 *            tree_attn_plan writes for these inputs, status codes included;
 *            a later layer's tree_attn_fwd can take anc_mask as its input.
 * Errors: the host checks of tree_attn_fwd, then the pointer rules of
 *   tree_attn_plan.  For a request with a non-zero status, out and lse rows
 *   are undefined (memory-safe), as after tree_attn_plan + tree_attn_fwd.
 */
ta_status_t tree_attn_plan_fwd(const void *q, const void *k_tree, const void *v_tree,
                               const void *k_cache, const void *v_cache,
                               const int32_t *block_table, const int32_t *prefix_len,
                               const int32_t *tree_off, const int32_t *parent,
                               int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t page_size, int32_t num_pages,
                               int32_t max_pages_per_seq, int32_t max_tree,
                               int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                               int32_t num_splits, uint64_t *anc_mask, int32_t *depth,
                               int32_t *pos_id, int32_t *status, void *out, float *lse,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * tree_attn_plan_dfs -- the plan, in a depth-first relabelling of each tree.
 *
 * The mask (JetFlow technical summary, section 2, tree-causal attention
 * mask) depends only on each node's root path, so any relabelling that
 * keeps parents before children changes no node's output.  This entry
 * relabels each request's forest in preorder, with the roots and each
 * node's children taken in increasing local index.  A node's ancestors then
 * sit just before it and every subtree is one contiguous range, so the
 * ancestor bits of neighbouring rows share 64-key blocks and more tree
 * blocks are skipped by tree_attn_fwd.
 *   parent, tree_off, prefix_len, B, N, max_tree: as tree_attn_plan.
 *   perm     [N] i32 (device, written): perm[off_b + i'] = off_b + i, the old
 *            global index of the node whose new local index is i'.
 *   inv_perm [N] i32: inv_perm[off_b + i] = off_b + i' (the inverse).
 *   parent_new [N] i32: the local parent of every node in the new labelling
 *            (parent_new[i'] < i').
 *   anc_mask, depth, pos_id, status: what tree_attn_plan writes for the
 *            relabelled tree (rows in the new order); the same status codes.
 * To run the attention in the new order, gather the rows of q, k_tree and
 * v_tree with perm (tree_attn_gather_rows) and call tree_attn_fwd with this
 * anc_mask; gathering its out and lse rows with inv_perm restores the old
 * order.  Outputs of a request with a non-zero status are undefined.
 * Errors, async behaviour and argument checks: as tree_attn_plan.
 */
ta_status_t tree_attn_plan_dfs(const int32_t *parent, const int32_t *tree_off,
                               const int32_t *prefix_len, int32_t B, int32_t N,
                               int32_t max_tree, int32_t *perm, int32_t *inv_perm,
                               int32_t *parent_new, uint64_t *anc_mask, int32_t *depth,
                               int32_t *pos_id, int32_t *status, void *stream);

/*
 * tree_attn_gather_rows -- dst[i] = src[index[i]] for n_rows rows of
 * row_bytes bytes each (device pointers).  It moves the rows of q, k_tree,
 * v_tree, out or lse between the old and the depth-first labelling of
 * tree_attn_plan_dfs; that the relabelled call gives the same outputs rests
 * on the mask depending only on root paths (JetFlow technical summary,
 * section 2, tree-causal attention mask).  An index outside [0, n_src) yields a zero row.
 * row_bytes must be a multiple of 4 and src, dst 4-byte aligned
 * (TA_ERR_BAD_SHAPE / TA_ERR_UNSUPPORTED).  src and dst must not overlap.
 * Enqueued on stream; returns without synchronising.
 */
ta_status_t tree_attn_gather_rows(const void *src, int64_t n_src, const int32_t *index, void *dst,
                                  int64_t n_rows, int64_t row_bytes, void *stream);

/*
 * tree_attn_build_tree -- best-first draft trees from per-depth candidates.
 *
 * The draft head produces logits for every tree depth in one pass; the
 * cumulative draft log-probability of a branch ranks the candidate nodes,
 * and best-first expansion grows each request's tree to the token budget
 * (JetFlow technical summary, section 2, tree construction).
 *   logp [B, max_depth, K] f32 (device): log-probability of candidate token k
 *        at depth d + 1, shared by every node at depth d; every value <= 0,
 *        -inf or NaN.  Positive values are outside the contract (the trees
 *        are built depth by depth on the fact that a child never beats its
 *        parent) and may differ from the expansion below.
 * Expansion: a virtual root (depth 0, score 0) pushes its K children (child
 * k: score logp[b, 0, k], push number k).  Then T times: pop the candidate
 * with the largest score, equal scores going to the smaller push number; it
 * becomes node i (i = 0, 1, ... in pop order); below max_depth it pushes its
 * K children, child k with score score_i + logp[b, depth_i, k] (one fp32
 * addition) and push number K + K*i + k.
 *   parent [B, T] i32 (device, written): parent node id (-1: hangs off the
 *          prefix); nodes are in pop order, so parent[i] < i and the trees
 *          can go to tree_attn_plan with tree_off[b] = b * T.
 *   choice [B, T] i32: the node's candidate index k at its depth.
 *   score  [B, T] f32: the node's cumulative log-probability.
 * Supported: K <= 64, max_depth <= 64, T <= 256, K * (T + 1) <= 16448,
 *   K * max_depth <= 4096; the implicit tree must hold T nodes
 *   (TA_ERR_BAD_SHAPE otherwise).  NaN log-probabilities are never chosen;
 *   if they leave fewer than T candidates, the missing nodes are written with
 *   parent -1, choice -1 and a NaN score.
 */
ta_status_t tree_attn_build_tree(const float *logp, int32_t B, int32_t max_depth, int32_t K,
                                 int32_t T, int32_t *parent, int32_t *choice, float *score,
                                 void *stream);

/*
 * tree_attn_commit -- append each request's accepted path to its paged cache.
 *
 * After verification the target model keeps the longest drafted branch it
 * agrees with and discards the rest (JetFlow technical summary, sections 1
 * and 4); the kept tokens join the context, so their keys and values join the
 * paged prefix.  For request b with accepted[b] = a (a local node id, or -1
 * when nothing was accepted), every node j on a's root path -- bit j of
 * anc_mask[tree_off[b] + a] -- is the token at position
 *   t = prefix_len[b] + depth[tree_off[b] + j] - 1,
 * and its K and V rows (all Hkv heads) are copied byte for byte from
 * k_tree / v_tree row tree_off[b] + j into k_cache / v_cache at page
 * block_table[b, t / page_size], slot t % page_size.  Then
 * new_prefix_len[b] = prefix_len[b] + depth[tree_off[b] + a].
 *
 * anc_mask, depth (device): as written by tree_attn_plan for these trees.
 * tree_off [B+1], prefix_len [B], accepted [B] i32 (device).
 * k_tree, v_tree [N, Hkv, D]; k_cache, v_cache [num_pages, page_size, Hkv, D]
 *   (device, dtype; all 16-byte aligned).  The caches are written in place.
 * block_table [B, max_pages_per_seq] i32 (device): must hold pages for the
 *   positions prefix_len[b] .. prefix_len[b] + depth(a) - 1.
 * new_prefix_len [B], status [B] i32 (device, written):
 *   status[b] = 0, TA_TREE_BAD_OFFSETS, TA_TREE_BAD_PREFIX,
 *   TA_COMMIT_BAD_ACCEPTED (a outside [-1, T_b)), TA_COMMIT_BAD_PAGE (a
 *   needed block-table entry is missing, beyond max_pages_per_seq or outside
 *   [0, num_pages)), or TA_COMMIT_BAD_PLAN (anc_mask / depth do not name one
 *   node per depth on a's path: they are not a plan of these trees).  On any
 *   non-zero status nothing of request b is written and new_prefix_len[b] =
 *   prefix_len[b].
 * Supported: dtype bf16 or fp32, Hkv * D * element size a multiple of 16
 *   bytes, page_size a power of two in [1, 1024], max_tree <= 256.
 * Requests must write disjoint cache slots (distinct pages); overlapping
 * writes land in an unspecified order.
 */
#define TA_COMMIT_BAD_ACCEPTED (-3)
#define TA_COMMIT_BAD_PAGE (-4)
#define TA_COMMIT_BAD_PLAN (-5)
ta_status_t tree_attn_commit(const uint64_t *anc_mask, const int32_t *depth, const int32_t *tree_off,
                             const int32_t *prefix_len, const int32_t *accepted, const void *k_tree,
                             const void *v_tree, void *k_cache, void *v_cache,
                             const int32_t *block_table, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                             int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq,
                             int32_t max_tree, ta_dtype_t dtype, int32_t *new_prefix_len,
                             int32_t *status, void *stream);

/*
 * The two stages of tree_attn_fwd, for callers that schedule or time them
 * separately.  Both take exactly the arguments of tree_attn_fwd and run the
 * same host checks; tree_attn_fwd is tree_attn_fwd_partial followed by
 * tree_attn_merge on the same stream.  Defined by: the tree-causal attention
 * of tree_attn_fwd (JetFlow technical summary, section 2, core architecture;
 * section 3, the paged prefix of the industrial integration).  Cutting the
 * prefix into chunks and merging their softmax by log-sum-exp rewrites the
 * same sums exactly; the pages state no split of their own.
 *   tree_attn_fwd_partial  launches the attention kernel.  With one prefix
 *                          split it writes out / lse itself; otherwise each
 *                          split writes its scaled partial output and its
 *                          (log-sum-exp, scale exponent) into the workspace.
 *   tree_attn_merge        combines the splits' partials into out / lse by
 *                          the log-sum-exp rule (split-K merge); a no-op
 *                          when there is one split.  It must follow the
 *                          partial stage of the same call, with the same
 *                          arguments and the workspace untouched.
 */
ta_status_t tree_attn_fwd_partial(const void *q, const void *k_tree, const void *v_tree,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *prefix_len,
                                  const int32_t *tree_off, const uint64_t *anc_mask,
                                  int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t page_size, int32_t num_pages,
                                  int32_t max_pages_per_seq, int32_t max_tree,
                                  int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                                  int32_t num_splits, void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream);

ta_status_t tree_attn_merge(const void *q, const void *k_tree, const void *v_tree,
                            const void *k_cache, const void *v_cache,
                            const int32_t *block_table, const int32_t *prefix_len,
                            const int32_t *tree_off, const uint64_t *anc_mask,
                            int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t page_size, int32_t num_pages,
                            int32_t max_pages_per_seq, int32_t max_tree,
                            int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                            int32_t num_splits, void *out, float *lse, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * The first stage of tree_attn_plan_fwd, with the same arguments and host
 * checks: the plan and the attention kernel (for fp32 or N = 0, the plan
 * kernel and tree_attn_fwd_partial).  Defined by: as tree_attn_plan_fwd
 * (JetFlow technical summary, section 2, tree-causal attention mask).  tree_attn_plan_fwd is this followed by
 * tree_attn_merge, called with the tree_attn_fwd arguments of the same call
 * (anc_mask = the mask output).
 */
ta_status_t tree_attn_plan_fwd_partial(const void *q, const void *k_tree, const void *v_tree,
                                       const void *k_cache, const void *v_cache,
                                       const int32_t *block_table, const int32_t *prefix_len,
                                       const int32_t *tree_off, const int32_t *parent,
                                       int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t page_size, int32_t num_pages,
                                       int32_t max_pages_per_seq, int32_t max_tree,
                                       int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                                       int32_t num_splits, uint64_t *anc_mask, int32_t *depth,
                                       int32_t *pos_id, int32_t *status, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * tree_attn_fwd_noalloc -- tree_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.
 *
 * The same operation, arguments, checks and results as tree_attn_fwd (bit for
 * bit), without the workspace arguments: the split workspace comes from a
 * fixed device array of TREE_ATTN_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per device, held until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's array address.
 * Limit: a call whose tree_attn_workspace_bytes(...) exceeds
 *   TREE_ATTN_NOALLOC_SCRATCH_BYTES returns TA_ERR_SCRATCH_LIMIT before
 *   anything is launched (budget 16, 64 and 256 trees of one to eight
 *   requests over prefixes of up to 8192 tokens fit; batches large enough
 *   to need no split use no workspace at all).
 * Every call on a device shares that device's array: calls that overlap on
 *   one device (different streams without ordering, or threads) race and
 *   give undefined results; order them.  The array keeps the last call's
 *   contents; no call depends on what an earlier call left there.
 */
#define TREE_ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
ta_status_t tree_attn_fwd_noalloc(const void *q, const void *k_tree, const void *v_tree,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *prefix_len,
                                  const int32_t *tree_off, const uint64_t *anc_mask,
                                  int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t page_size, int32_t num_pages,
                                  int32_t max_pages_per_seq, int32_t max_tree,
                                  int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                                  int32_t num_splits, void *out, float *lse, void *stream);

/*
 * The host-side argument check of tree_attn_fwd, on its own: returns exactly
 * what tree_attn_fwd would return before launching anything (TA_OK if it
 * would launch).  Launches nothing and touches no device memory.
 */
ta_status_t tree_attn_fwd_check(const void *q, const void *k_tree, const void *v_tree,
                                const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *prefix_len,
                                const int32_t *tree_off, const uint64_t *anc_mask,
                                int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t page_size, int32_t num_pages,
                                int32_t max_pages_per_seq, int32_t max_tree,
                                int32_t max_prefix, float softmax_scale, ta_dtype_t dtype,
                                int32_t num_splits, const void *out, const float *lse,
                                const void *workspace, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
