/*
 * Plain fp64 CPU oracle for tree-causal paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the HIP library: it is written directly from the definition of
 * the operation, as slowly and plainly as that definition reads.
 *
 * What it computes (JetFlow technical summary, section 2 "core architecture",
 * tree-causal attention mask; the same paragraph on the French page):
 *   every node of a draft token tree attends to the original input prefix and
 *   to its own ancestors inside the tree -- never to its descendants and never
 *   to unrelated sibling branches.  The branch factorisation printed right
 *   below it, q(pi(v)|x) = prod_{u in pi(v)} q(y_u | x, h, pi_{<u}), conditions
 *   the token at node u on the prefix and on the path before u, so the token
 *   at u is produced at u itself: the node's own key is visible (a node is on
 *   its own root-to-node path).
 * The prefix lives in a paged KV cache (the verification kernel of the same
 * pages, section 3 "industrial integration", is a paged FlashAttention with
 * tree-mask staging), addressed through a per-request block table.
 *
 * For request b, local node i, query head h (kv head c = h / (Hq/Hkv)):
 *   visible keys  = { prefix t : 0 <= t < L_b }  U  { tree j : j on the path
 *                   from i up to its root, found by following parent[] }
 *   s_k   = scale * <q[i,h], K_k>
 *   m     = max_k s_k,   l = sum_k exp(s_k - m)
 *   O     = sum_k exp(s_k - m) V_k / l,     LSE = m + ln l   (natural log)
 * all in fp64 on the exact input values.
 *
 * The plan outputs (ancestor bitmask, depth, position id) are computed the
 * same way, by walking parent pointers: bit j of node i's mask is set iff j is
 * on i's root path (i included), depth = number of such nodes, and
 * pos_id = L_b + depth - 1 is the position the node would have in the flat
 * sequence prefix ++ path.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MASK_WORDS 4
#define ORACLE_MAX_TREE (64 * ORACLE_MASK_WORDS)

/* per-request status codes of the plan (same contract as the library's) */
#define ORACLE_TREE_OK 0
#define ORACLE_TREE_BAD_OFFSETS (-1)
#define ORACLE_TREE_BAD_PREFIX (-2)

/* return codes of oracle_tree_attn */
#define ORACLE_OK 0
#define ORACLE_ERR_ARGS 1
#define ORACLE_ERR_TREE 2
#define ORACLE_ERR_PAGE 3
#define ORACLE_ERR_ALLOC 4

/*
 * Plan for every request b, written one node at a time:
 *   status[b] = -1 if the offsets are inconsistent (tree_off[0] != 0,
 *               tree_off[B] != N, a negative tree size, or a tree larger than
 *               max_tree), else -2 if prefix_len[b] < 0, else k > 0 if node
 *               k-1 is the first node whose parent is not in [-1, k-2], else 0.
 * Rows of requests with a non-zero status are zero-filled.
 */
int oracle_plan(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                int32_t B, int32_t N, int32_t max_tree,
                uint64_t *anc_mask, int32_t *depth, int32_t *pos_id, int32_t *status)
{
    if (B < 0 || N < 0 || max_tree < 0 || max_tree > ORACLE_MAX_TREE)
        return ORACLE_ERR_ARGS;
    for (int64_t n = 0; n < (int64_t)N * ORACLE_MASK_WORDS; ++n)
        anc_mask[n] = 0;
    for (int32_t n = 0; n < N; ++n) {
        depth[n] = 0;
        pos_id[n] = 0;
    }
    for (int32_t b = 0; b < B; ++b) {
        int32_t off = tree_off[b], end = tree_off[b + 1];
        int32_t T = end - off;
        int bad_offsets = (T < 0) || (T > max_tree) || (off < 0) || (end > N) ||
                          (b == 0 && off != 0) || (b == B - 1 && end != N);
        if (bad_offsets) {
            status[b] = ORACLE_TREE_BAD_OFFSETS;
            continue;
        }
        if (prefix_len[b] < 0) {
            status[b] = ORACLE_TREE_BAD_PREFIX;
            continue;
        }
        int32_t first_bad = -1;
        for (int32_t i = 0; i < T; ++i) {
            int32_t p = parent[off + i];
            if (p < -1 || p >= i) {
                first_bad = i;
                break;
            }
        }
        if (first_bad >= 0) {
            status[b] = first_bad + 1;
            continue;
        }
        for (int32_t i = 0; i < T; ++i) {
            int32_t d = 0;
            /* walk i, parent(i), parent(parent(i)), ... until -1 */
            for (int32_t j = i; j != -1; j = parent[off + j]) {
                anc_mask[(int64_t)(off + i) * ORACLE_MASK_WORDS + j / 64] |= (uint64_t)1 << (j % 64);
                d += 1;
            }
            depth[off + i] = d;
            pos_id[off + i] = prefix_len[b] + d - 1;
        }
        status[b] = ORACLE_TREE_OK;
    }
    return ORACLE_OK;
}

/*
 * Depth-first relabelling of every request's tree (the pages define only the
 * mask, JetFlow technical summary, section 2: a node sees its own root path;
 * any relabelling that keeps parents before children leaves every node's
 * output unchanged).  The order is the preorder of the forest with the roots,
 * and each node's children, taken in increasing local index, written with an
 * explicit stack:
 *   perm[off + i'] = off + i   (new local index i' of old node i)
 *   inv[off + i]   = off + i'
 *   parent_new[off + i'] = new index of parent(i), or -1 for a root.
 * The status is the plan's (same checks, same codes).  Rows of requests with
 * a non-zero status get the identity and their parent array unchanged.
 */
int oracle_dfs_order(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                     int32_t B, int32_t N, int32_t max_tree,
                     int32_t *perm, int32_t *inv, int32_t *parent_new, int32_t *status)
{
    if (B < 0 || N < 0 || max_tree < 0 || max_tree > ORACLE_MAX_TREE)
        return ORACLE_ERR_ARGS;
    for (int32_t n = 0; n < N; ++n) {
        perm[n] = n;
        inv[n] = n;
        parent_new[n] = parent[n];
    }
    int32_t stack[ORACLE_MAX_TREE];
    for (int32_t b = 0; b < B; ++b) {
        int32_t off = tree_off[b], end = tree_off[b + 1];
        int32_t T = end - off;
        int bad_offsets = (T < 0) || (T > max_tree) || (off < 0) || (end > N) ||
                          (b == 0 && off != 0) || (b == B - 1 && end != N);
        if (bad_offsets) {
            status[b] = ORACLE_TREE_BAD_OFFSETS;
            continue;
        }
        if (prefix_len[b] < 0) {
            status[b] = ORACLE_TREE_BAD_PREFIX;
            continue;
        }
        int32_t first_bad = -1;
        for (int32_t i = 0; i < T; ++i) {
            int32_t p = parent[off + i];
            if (p < -1 || p >= i) {
                first_bad = i;
                break;
            }
        }
        if (first_bad >= 0) {
            status[b] = first_bad + 1;
            continue;
        }
        /* Depth-first walk.  The stack holds nodes still to visit; the
         * children of a node (and the roots) are pushed largest index first,
         * so that they come off in increasing index order.  Every node is
         * pushed exactly once, by its parent (or as a root). */
        int32_t top = 0, next = 0;
        for (int32_t i = T - 1; i >= 0; --i)
            if (parent[off + i] == -1)
                stack[top++] = i;
        while (top > 0) {
            int32_t v = stack[--top];
            perm[off + next] = off + v;
            inv[off + v] = off + next;
            next += 1;
            for (int32_t c = T - 1; c > v; --c)
                if (parent[off + c] == v)
                    stack[top++] = c;
        }
        for (int32_t i = 0; i < T; ++i) {
            int32_t p = parent[off + i];
            parent_new[inv[off + i]] = (p == -1) ? -1 : inv[off + p] - off;
        }
        status[b] = ORACLE_TREE_OK;
    }
    return ORACLE_OK;
}

typedef struct {
    const double *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len, *tree_off, *parent;
    int32_t B, N, Hq, Hkv, D, page_size, max_pages, num_pages;
    double scale;
    const int64_t *rows; /* NULL: every (node, head) row */
    int64_t n_rows;
    double *out, *lse;
    int64_t next;        /* work counter, taken with an atomic add */
    int error;
    int32_t max_keys;
} oracle_job;

static int32_t request_of(const int32_t *tree_off, int32_t B, int32_t node)
{
    for (int32_t b = 0; b < B; ++b)
        if (node >= tree_off[b] && node < tree_off[b + 1])
            return b;
    return -1;
}

static double dot(const double *a, const double *b, int32_t D)
{
    double s = 0.0;
    for (int32_t d = 0; d < D; ++d)
        s += a[d] * b[d];
    return s;
}

/* One query row (node, head): returns 0 or an ORACLE_ERR_* code. */
static int one_row(const oracle_job *J, int32_t node, int32_t h, double *o, double *lse,
                   double *score, const double **vrow)
{
    int32_t b = request_of(J->tree_off, J->B, node);
    if (b < 0)
        return ORACLE_ERR_ARGS;
    int32_t off = J->tree_off[b];
    int32_t T = J->tree_off[b + 1] - off;
    int32_t i = node - off;
    int32_t L = J->prefix_len[b];
    int32_t G = J->Hq / J->Hkv;
    int32_t c = h / G;
    int32_t D = J->D;
    const double *qrow = J->q + ((int64_t)node * J->Hq + h) * D;
    int32_t n = 0;

    /* the prefix, through the block table */
    for (int32_t t = 0; t < L; ++t) {
        int32_t page = J->block_table[(int64_t)b * J->max_pages + t / J->page_size];
        if (page < 0 || page >= J->num_pages)
            return ORACLE_ERR_PAGE;
        int64_t slot = (int64_t)page * J->page_size + t % J->page_size;
        const double *krow = J->k_cache + (slot * J->Hkv + c) * D;
        score[n] = J->scale * dot(qrow, krow, D);
        vrow[n] = J->v_cache + (slot * J->Hkv + c) * D;
        n += 1;
    }
    /* the node itself and its ancestors, by walking parent pointers */
    int32_t steps = 0;
    for (int32_t j = i; j != -1; j = J->parent[off + j]) {
        if (j < 0 || j >= T || steps > T)
            return ORACLE_ERR_TREE;
        int32_t p = J->parent[off + j];
        if (p < -1 || p >= j)
            return ORACLE_ERR_TREE;
        const double *krow = J->k_tree + ((int64_t)(off + j) * J->Hkv + c) * D;
        score[n] = J->scale * dot(qrow, krow, D);
        vrow[n] = J->v_tree + ((int64_t)(off + j) * J->Hkv + c) * D;
        n += 1;
        steps += 1;
    }

    double m = -INFINITY;
    for (int32_t k = 0; k < n; ++k)
        if (score[k] > m)
            m = score[k];
    double l = 0.0;
    for (int32_t k = 0; k < n; ++k)
        l += exp(score[k] - m);
    for (int32_t d = 0; d < D; ++d)
        o[d] = 0.0;
    for (int32_t k = 0; k < n; ++k) {
        double w = exp(score[k] - m) / l;
        for (int32_t d = 0; d < D; ++d)
            o[d] += w * vrow[k][d];
    }
    *lse = m + log(l);
    return ORACLE_OK;
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *score = (double *)malloc(sizeof(double) * (size_t)J->max_keys);
    const double **vrow = (const double **)malloc(sizeof(double *) * (size_t)J->max_keys);
    if (!score || !vrow) {
        __atomic_store_n(&J->error, ORACLE_ERR_ALLOC, __ATOMIC_RELAXED);
        free(score);
        free((void *)vrow);
        return NULL;
    }
    int64_t total = J->rows ? J->n_rows : (int64_t)J->N * J->Hq;
    for (;;) {
        int64_t r = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (r >= total)
            break;
        int64_t row = J->rows ? J->rows[r] : r;
        int32_t node = (int32_t)(row / J->Hq), h = (int32_t)(row % J->Hq);
        int rc = one_row(J, node, h, J->out + r * J->D, J->lse + r, score, vrow);
        if (rc != ORACLE_OK)
            __atomic_store_n(&J->error, rc, __ATOMIC_RELAXED);
    }
    free(score);
    free((void *)vrow);
    return NULL;
}

/*
 * Tree attention for every (node, q-head) row, or for the listed rows only
 * (row = node * Hq + h).  Layouts, all row-major:
 *   q [N,Hq,D], k_tree/v_tree [N,Hkv,D], k_cache/v_cache
 *   [num_pages,page_size,Hkv,D], block_table [B,max_pages], tree_off [B+1],
 *   prefix_len [B], parent [N] (local ids, -1 = root).
 * Output: out [R,D] and lse [R] with R = n_rows, or N*Hq when rows == NULL.
 */
int oracle_tree_attn(const double *q, const double *k_tree, const double *v_tree,
                     const double *k_cache, const double *v_cache,
                     const int32_t *block_table, const int32_t *prefix_len,
                     const int32_t *tree_off, const int32_t *parent,
                     int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                     int32_t page_size, int32_t max_pages, int32_t num_pages, double scale,
                     const int64_t *rows, int64_t n_rows,
                     double *out, double *lse, int32_t n_threads)
{
    if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || page_size <= 0)
        return ORACLE_ERR_ARGS;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k_tree = k_tree; J.v_tree = v_tree; J.k_cache = k_cache; J.v_cache = v_cache;
    J.block_table = block_table; J.prefix_len = prefix_len; J.tree_off = tree_off; J.parent = parent;
    J.B = B; J.N = N; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.page_size = page_size;
    J.max_pages = max_pages; J.num_pages = num_pages; J.scale = scale;
    J.rows = rows; J.n_rows = n_rows; J.out = out; J.lse = lse;
    int32_t maxL = 0, maxT = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (prefix_len[b] < 0 || (int64_t)prefix_len[b] > (int64_t)max_pages * page_size)
            return ORACLE_ERR_ARGS;
        if (prefix_len[b] > maxL) maxL = prefix_len[b];
        if (tree_off[b + 1] - tree_off[b] > maxT) maxT = tree_off[b + 1] - tree_off[b];
    }
    J.max_keys = maxL + maxT + 1;
    if (n_threads < 1)
        n_threads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th)
        return ORACLE_ERR_ALLOC;
    int32_t started = 0;
    for (int32_t t = 0; t < n_threads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &J) != 0)
            break;
        started += 1;
    }
    if (started == 0)
        worker(&J);
    for (int32_t t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    free(th);
    return J.error;
}

/*
 * Commit of the accepted path (the step after verification: JetFlow
 * technical summary, section 4 and section 1 -- the target model keeps the
 * longest drafted branch it agrees with and throws the other guesses away; the
 * kept tokens join the context, so their keys and values join the paged
 * prefix cache).
 *
 * For request b with accepted[b] = a (a local node id, or -1 when nothing was
 * accepted): the path is a's root path, root first, found by following
 * parent[] up from a.  The node at depth d (1-based) is the token at position
 * t = L_b + d - 1 of the sequence, so its K and V rows (all Hkv heads) are
 * copied byte for byte from k_tree / v_tree row tree_off[b] + node into
 * k_cache / v_cache at page block_table[b][t / page_size], slot
 * t % page_size.  new_prefix_len[b] = L_b + depth(a).
 *
 * status[b] (checked in this order; on any failure nothing of request b is
 * written and new_prefix_len[b] = prefix_len[b]):
 *   -1 bad offsets (as the plan), -2 prefix_len[b] < 0,
 *   -3 accepted[b] outside [-1, T_b),
 *   k > 0: node k-1 on the path has a parent outside [-1, k-1),
 *   -4 a block-table entry for one of the positions L_b .. L_b + depth - 1
 *      lies beyond max_pages or names a page outside [0, num_pages).
 * Rows are elem_size * Hkv * D bytes.  Returns ORACLE_ERR_ARGS for bad sizes.
 */
#define ORACLE_COMMIT_BAD_ACCEPTED (-3)
#define ORACLE_COMMIT_BAD_PAGE (-4)

int oracle_commit(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                  const int32_t *accepted, const void *k_tree, const void *v_tree, void *k_cache,
                  void *v_cache, const int32_t *block_table, int32_t B, int32_t N, int32_t Hkv,
                  int32_t D, int32_t elem_size, int32_t page_size, int32_t num_pages,
                  int32_t max_pages, int32_t max_tree, int32_t *new_prefix_len, int32_t *status)
{
    if (B < 0 || N < 0 || Hkv < 1 || D < 1 || elem_size < 1 || page_size < 1 || num_pages < 0 ||
        max_pages < 0 || max_tree < 0 || max_tree > ORACLE_MAX_TREE)
        return ORACLE_ERR_ARGS;
    const size_t row_bytes = (size_t)elem_size * (size_t)Hkv * (size_t)D;
    int32_t path[ORACLE_MAX_TREE];
    for (int32_t b = 0; b < B; ++b) {
        const int32_t off = tree_off[b];
        const int32_t end = tree_off[b + 1];
        const int32_t T = end - off;
        const int32_t L = prefix_len[b];
        new_prefix_len[b] = L;
        if (T < 0 || T > max_tree || off < 0 || end > N || (b == 0 && off != 0) ||
            (b == B - 1 && end != N)) {
            status[b] = ORACLE_TREE_BAD_OFFSETS;
            continue;
        }
        if (L < 0) {
            status[b] = ORACLE_TREE_BAD_PREFIX;
            continue;
        }
        const int32_t a = accepted[b];
        if (a < -1 || a >= T) {
            status[b] = ORACLE_COMMIT_BAD_ACCEPTED;
            continue;
        }
        /* walk up from a, recording the path leaf first */
        int32_t depth = 0, bad = 0;
        for (int32_t i = a; i >= 0;) {
            const int32_t p = parent[off + i];
            if (p < -1 || p >= i) {
                bad = i + 1;
                break;
            }
            path[depth++] = i;
            i = p;
        }
        if (bad) {
            status[b] = bad;
            continue;
        }
        /* every page the path's positions land in must exist */
        for (int32_t d = 0; d < depth; ++d) {
            const int64_t t = (int64_t)L + d;
            const int64_t slot_page = t / page_size;
            if (slot_page >= max_pages) {
                bad = 1;
                break;
            }
            const int32_t page = block_table[(int64_t)b * max_pages + slot_page];
            if (page < 0 || page >= num_pages) {
                bad = 1;
                break;
            }
        }
        if (bad) {
            status[b] = ORACLE_COMMIT_BAD_PAGE;
            continue;
        }
        /* copy root first: the node at depth d is path[depth - d] */
        for (int32_t d = 1; d <= depth; ++d) {
            const int32_t node = path[depth - d];
            const int64_t t = (int64_t)L + d - 1;
            const int32_t page = block_table[(int64_t)b * max_pages + t / page_size];
            const int64_t dst_row = (int64_t)page * page_size + t % page_size;
            const int64_t src_row = (int64_t)off + node;
            memcpy((char *)k_cache + dst_row * row_bytes, (const char *)k_tree + src_row * row_bytes, row_bytes);
            memcpy((char *)v_cache + dst_row * row_bytes, (const char *)v_tree + src_row * row_bytes, row_bytes);
        }
        new_prefix_len[b] = L + depth;
        status[b] = ORACLE_TREE_OK;
    }
    return ORACLE_OK;
}

/*
 * Draft-tree construction (JetFlow technical summary, section 2, training
 * strategy / tree construction: the draft head produces logits for every
 * tree depth in one pass, a branch score -- by default the cumulative draft
 * log-probability -- ranks the candidate nodes, and best-first expansion
 * grows the tree until the token budget is reached).
 *
 * Input per request b: logp[b][d][k] (fp32), the log-probability of candidate
 * token k (0 <= k < K) at depth d + 1 (0 <= d < Dmax), shared by every node at
 * depth d (the literal reading: one draft distribution per depth).
 * Best-first, in steps:
 *   1. a virtual root at depth 0 with score 0 pushes its K children: child k
 *      has score logp[0][k] and push number k;
 *   2. T times: pop the candidate with the largest score (equal scores: the
 *      smaller push number); it becomes node i (i = 0, 1, ... in pop order),
 *      with parent = the node that pushed it (-1 for the root), choice = its
 *      k, score = its score; if its depth is below Dmax it pushes its K
 *      children: child k has score score_i + logp[depth_i][k] (one fp32
 *      addition) and push number K + K * i + k.
 * Outputs per request: parent, choice, score for nodes 0 .. T-1 at offset
 * b * T.  Scores are fp32 sums taken in this order, so any implementation
 * that adds in the same order decides every comparison identically.
 * T must not exceed the number of nodes of the implicit tree.
 * NaN log-probabilities (outside the pages' definition, which ranks real
 * scores) are read as "no candidate": a candidate with a NaN score is never
 * pushed, so it is never popped; when the pool runs dry before T pops, the
 * remaining nodes are written as missing (parent -1, choice -1, NaN score).
 */
typedef struct {
    float score;
    int64_t push;
    int32_t parent, depth, k;
} cand_t;

static int cand_before(const cand_t *a, const cand_t *b)
{
    /* a pops before b */
    if (a->score != b->score)
        return a->score > b->score;
    return a->push < b->push;
}

static void heap_push(cand_t *h, int64_t *n, cand_t c)
{
    int64_t i = (*n)++;
    h[i] = c;
    while (i > 0) {
        int64_t up = (i - 1) / 2;
        if (!cand_before(&h[i], &h[up]))
            break;
        cand_t t = h[i];
        h[i] = h[up];
        h[up] = t;
        i = up;
    }
}

static cand_t heap_pop(cand_t *h, int64_t *n)
{
    cand_t top = h[0];
    h[0] = h[--(*n)];
    int64_t i = 0;
    for (;;) {
        int64_t l = 2 * i + 1, r = l + 1, m = i;
        if (l < *n && cand_before(&h[l], &h[m]))
            m = l;
        if (r < *n && cand_before(&h[r], &h[m]))
            m = r;
        if (m == i)
            break;
        cand_t t = h[i];
        h[i] = h[m];
        h[m] = t;
        i = m;
    }
    return top;
}

int oracle_build_tree(const float *logp, int32_t B, int32_t Dmax, int32_t K, int32_t T,
                      int32_t *parent, int32_t *choice, float *score)
{
    if (B < 0 || Dmax < 1 || K < 1 || T < 0)
        return ORACLE_ERR_ARGS;
    /* the implicit tree must hold T nodes */
    double nodes = 0, level = 1;
    for (int32_t d = 0; d < Dmax && nodes < T; ++d) {
        level *= K;
        nodes += level;
    }
    if (nodes < T)
        return ORACLE_ERR_ARGS;
    const int64_t cap = (int64_t)K * (T + 1) + 1;
    cand_t *h = (cand_t *)malloc(sizeof(cand_t) * (size_t)cap);
    if (!h)
        return ORACLE_ERR_ALLOC;
    for (int32_t b = 0; b < B; ++b) {
        const float *lp = logp + (int64_t)b * Dmax * K;
        int64_t n = 0;
        for (int32_t k = 0; k < K; ++k) {
            cand_t c = {lp[k], k, -1, 1, k};
            if (c.score == c.score)
                heap_push(h, &n, c);
        }
        for (int32_t i = 0; i < T; ++i) {
            if (n == 0) {
                /* no candidate left: the node is missing */
                parent[(int64_t)b * T + i] = -1;
                choice[(int64_t)b * T + i] = -1;
                score[(int64_t)b * T + i] = NAN;
                continue;
            }
            const cand_t c = heap_pop(h, &n);
            parent[(int64_t)b * T + i] = c.parent;
            choice[(int64_t)b * T + i] = c.k;
            score[(int64_t)b * T + i] = c.score;
            if (c.depth < Dmax) {
                for (int32_t k = 0; k < K; ++k) {
                    volatile float s = c.score + lp[(int64_t)c.depth * K + k];
                    cand_t ch = {s, (int64_t)K + (int64_t)K * i + k, i, c.depth + 1, k};
                    if (ch.score == ch.score)
                        heap_push(h, &n, ch);
                }
            }
        }
    }
    free(h);
    return ORACLE_OK;
}
