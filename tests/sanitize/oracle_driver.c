/* Host driver for the oracle under AddressSanitizer and UndefinedBehaviour-
 * Sanitizer: every oracle entry point on small seeded inputs, valid and
 * invalid, with light consistency checks.  Exits non-zero on a failed check;
 * the sanitizers abort on any memory or UB error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_plan(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len, int32_t B,
                int32_t N, int32_t max_tree, uint64_t *anc_mask, int32_t *depth, int32_t *pos_id,
                int32_t *status);
int oracle_dfs_order(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len, int32_t B,
                     int32_t N, int32_t max_tree, int32_t *perm, int32_t *inv, int32_t *parent_new,
                     int32_t *status);
int oracle_tree_attn(const double *q, const double *k_tree, const double *v_tree, const double *k_cache,
                     const double *v_cache, const int32_t *block_table, const int32_t *prefix_len,
                     const int32_t *tree_off, const int32_t *parent, int32_t B, int32_t N, int32_t Hq,
                     int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages, int32_t num_pages,
                     double scale, const int64_t *rows, int64_t n_rows, double *out, double *lse,
                     int32_t n_threads);
int oracle_commit(const int32_t *parent, const int32_t *tree_off, const int32_t *prefix_len,
                  const int32_t *accepted, const void *k_tree, const void *v_tree, void *k_cache,
                  void *v_cache, const int32_t *block_table, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                  int32_t elem_size, int32_t page_size, int32_t num_pages, int32_t max_pages,
                  int32_t max_tree, int32_t *new_prefix_len, int32_t *status);
int oracle_build_tree(const float *logp, int32_t B, int32_t Dmax, int32_t K, int32_t T, int32_t *parent,
                      int32_t *choice, float *score);

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint64_t lcg = 12345;
static double urand(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) / 9007199254740992.0;
}

enum { B = 3, N = 19, HQ = 4, HKV = 2, D = 8, PS = 4, MAXP = 13, NPAGES = 40, MAXT = 8 };

int main(void)
{
    /* request 0: chain of 5, prefix 0; request 1: a forest of 6, prefix 17;
     * request 2: a tree of 8, prefix 40 */
    const int32_t parent[N] = {-1, 0, 1, 2, 3, -1, -1, 0, 1, 0, -1, -1, 0, 0, 1, 2, 2, 4, 5};
    const int32_t tree_off[B + 1] = {0, 5, 11, 19};
    const int32_t prefix_len[B] = {0, 17, 40};
    int32_t bt[B * MAXP];
    for (int i = 0; i < B * MAXP; ++i)
        bt[i] = -1;
    int next = 0;
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < (prefix_len[b] + MAXT + PS - 1) / PS; ++p)
            bt[b * MAXP + p] = (next++ * 7) % NPAGES;   /* scattered pages, room to commit */

    uint64_t mask[N * 4];
    int32_t depth[N], pos[N], status[B];
    CHECK(oracle_plan(parent, tree_off, prefix_len, B, N, MAXT, mask, depth, pos, status) == 0);
    for (int b = 0; b < B; ++b)
        CHECK(status[b] == 0);
    for (int n = 0; n < N; ++n) {
        int pc = 0;
        for (int w = 0; w < 4; ++w)
            pc += __builtin_popcountll(mask[n * 4 + w]);
        CHECK(pc == depth[n]);
    }

    size_t qn = (size_t)N * HQ * D, tn = (size_t)N * HKV * D, cn = (size_t)NPAGES * PS * HKV * D;
    double *q = malloc(qn * sizeof(double)), *kt = malloc(tn * sizeof(double)), *vt = malloc(tn * sizeof(double));
    double *kc = malloc(cn * sizeof(double)), *vc = malloc(cn * sizeof(double));
    for (size_t i = 0; i < qn; ++i) q[i] = urand() * 2 - 1;
    for (size_t i = 0; i < tn; ++i) { kt[i] = urand() * 2 - 1; vt[i] = urand() * 2 - 1; }
    for (size_t i = 0; i < cn; ++i) { kc[i] = urand() * 2 - 1; vc[i] = urand() * 2 - 1; }
    double *out1 = malloc(qn * sizeof(double)), *out3 = malloc(qn * sizeof(double));
    double lse1[N * HQ], lse3[N * HQ];
    CHECK(oracle_tree_attn(q, kt, vt, kc, vc, bt, prefix_len, tree_off, parent, B, N, HQ, HKV, D, PS, MAXP,
                           NPAGES, 0.0, NULL, (int64_t)N * HQ, out1, lse1, 1) == 0);
    CHECK(oracle_tree_attn(q, kt, vt, kc, vc, bt, prefix_len, tree_off, parent, B, N, HQ, HKV, D, PS, MAXP,
                           NPAGES, 0.0, NULL, (int64_t)N * HQ, out3, lse3, 3) == 0);
    CHECK(memcmp(out1, out3, qn * sizeof(double)) == 0);
    for (int r = 0; r < N * HQ; ++r)
        CHECK(isfinite(lse1[r]));
    /* a row subset gives the same rows */
    int64_t rows[5] = {0, 7, 33, 60, N * HQ - 1};
    double outr[5 * D], lser[5];
    CHECK(oracle_tree_attn(q, kt, vt, kc, vc, bt, prefix_len, tree_off, parent, B, N, HQ, HKV, D, PS, MAXP,
                           NPAGES, 0.25, rows, 5, outr, lser, 2) == 0);
    /* bad inputs are refused, not read out of bounds */
    int32_t bad_parent[N];
    memcpy(bad_parent, parent, sizeof bad_parent);
    bad_parent[7] = 9;
    CHECK(oracle_plan(bad_parent, tree_off, prefix_len, B, N, MAXT, mask, depth, pos, status) == 0);
    CHECK(status[1] == 3);
    const int32_t bad_off[B + 1] = {0, 5, 21, 19};
    CHECK(oracle_plan(parent, bad_off, prefix_len, B, N, MAXT, mask, depth, pos, status) == 0);
    CHECK(status[1] == -1);

    int32_t perm[N], inv[N], pnew[N];
    CHECK(oracle_dfs_order(parent, tree_off, prefix_len, B, N, MAXT, perm, inv, pnew, status) == 0);
    for (int n = 0; n < N; ++n)
        CHECK(inv[perm[n]] == n);

    /* commit the deepest node of each request into byte copies of the caches */
    int32_t accepted[B] = {4, 3, 7}, newlen[B];
    CHECK(oracle_commit(parent, tree_off, prefix_len, accepted, kt, vt, kc, vc, bt, B, N, HKV, D,
                        (int32_t)sizeof(double), PS, NPAGES, MAXP, MAXT, newlen, status) == 0);
    CHECK(newlen[0] == 5 && status[0] == 0);
    int32_t acc_bad[B] = {5, -1, 8};
    CHECK(oracle_commit(parent, tree_off, prefix_len, acc_bad, kt, vt, kc, vc, bt, B, N, HKV, D,
                        (int32_t)sizeof(double), PS, NPAGES, MAXP, MAXT, newlen, status) == 0);
    CHECK(status[0] != 0 && status[1] == 0 && newlen[1] == prefix_len[1]);

    /* best-first trees, with ties and NaN candidates */
    float logp[2 * 4 * 3];
    for (int i = 0; i < 24; ++i)
        logp[i] = (float)(-urand() * 3);
    logp[2] = logp[1];
    logp[13] = NAN;
    int32_t tp[2 * 10], tc[2 * 10];
    float ts[2 * 10];
    CHECK(oracle_build_tree(logp, 2, 4, 3, 10, tp, tc, ts) == 0);
    for (int i = 0; i < 20; ++i)
        CHECK(tp[i] < i % 10);

    free(q); free(kt); free(vt); free(kc); free(vc); free(out1); free(out3);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
