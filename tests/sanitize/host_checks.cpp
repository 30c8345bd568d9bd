// Host dispatch (tree_attn.cpp) under AddressSanitizer and UndefinedBehaviour-
// Sanitizer, with the kernel launchers replaced by stubs that record their
// parameters: every extern "C" entry point is called with valid and invalid
// arguments (pointers are never dereferenced on the host), return codes are
// checked, and the workspace regions handed to the attention kernels must
// lie inside the caller's workspace.  Exits non-zero on a failed check.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "launch.h"
#include "tree_attn.h"

namespace ta {
static int n_launch = 0;
static FwdParams last_fwd;
hipError_t launch_plan(const PlanParams &, hipStream_t) { ++n_launch; return hipSuccess; }
hipError_t launch_plan_dfs(const PlanDfsParams &, hipStream_t) { ++n_launch; return hipSuccess; }
hipError_t launch_gather(const GatherParams &, hipStream_t) { ++n_launch; return hipSuccess; }
hipError_t launch_build_tree(const TreeParams &, hipStream_t) { ++n_launch; return hipSuccess; }
hipError_t launch_commit(const CommitParams &, hipStream_t) { ++n_launch; return hipSuccess; }
hipError_t launch_fwd(const FwdParams &p, int, int, int, int, hipStream_t)
{
    ++n_launch;
    last_fwd = p;
    return hipSuccess;
}
hipError_t launch_merge(const FwdParams &, hipStream_t) { ++n_launch; return hipSuccess; }
}  // namespace ta

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

// fake device addresses: distinct, aligned, never dereferenced
static void *fake(size_t i) { return (void *)(uintptr_t)(0x100000000ull + i * 0x1000000ull); }

struct Shape {
    int B, N, Hq, Hkv, D, ps, pages, maxp, maxt, maxpre;
};

static ta_status_t fwd(const Shape &s, ta_dtype_t dt, int splits, void *ws, size_t wsb, bool null_q = false)
{
    return tree_attn_fwd(null_q ? nullptr : fake(1), fake(2), fake(3), fake(4), fake(5), (const int32_t *)fake(6),
                         (const int32_t *)fake(7), (const int32_t *)fake(8), (const uint64_t *)fake(9), s.B, s.N,
                         s.Hq, s.Hkv, s.D, s.ps, s.pages, s.maxp, s.maxt, s.maxpre, 0.f, dt, splits, fake(10),
                         (float *)fake(11), ws, wsb, nullptr);
}

int main()
{
    const Shape shapes[] = {
        {1, 16, 32, 8, 128, 16, 150, 128, 16, 2048},     // budget 16
        {1, 256, 32, 8, 128, 16, 150, 128, 256, 2048},   // budget 256, one request
        {8, 512, 32, 8, 128, 16, 2400, 512, 64, 8192},   // mixed batch
        {32, 8192, 32, 4, 128, 16, 9100, 256, 256, 4096},
        {1, 16, 4, 1, 64, 16, 9, 8, 16, 128},
        {3, 40, 10, 2, 64, 1, 400, 300, 20, 300},
        {2, 7, 8, 2, 128, 1024, 3, 2, 5, 2000},
    };
    for (const Shape &s : shapes) {
        for (ta_dtype_t dt : {TA_DTYPE_BF16, TA_DTYPE_FP32}) {
            for (int splits : {0, 1, 2, 5, 17, 64}) {
                const size_t need = tree_attn_workspace_bytes(s.B, s.N, s.Hq, s.Hkv, s.D, s.maxt, s.maxpre, dt, splits);
                std::vector<char> host_ws(need + 512);
                // a 256-aligned address inside the vector, so that the
                // pointer arithmetic below is checked against real bounds
                char *ws = need ? (char *)(((uintptr_t)host_ws.data() + 255) & ~(uintptr_t)255) : nullptr;
                const int before = ta::n_launch;
                const ta_status_t st = fwd(s, dt, splits, ws, need);
                CHECK(st == TA_OK);
                CHECK(ta::n_launch > before);
                const ta::FwdParams &p = ta::last_fwd;
                if (dt == TA_DTYPE_BF16 && p.nsplit > 1) {
                    CHECK(need > 0);
                    const char *o0 = (const char *)p.ws_o;
                    const char *l0 = (const char *)p.ws_ml;
                    CHECK(o0 >= ws && o0 + (size_t)p.nsplit * s.N * s.Hq * s.D * 2 <= l0);
                    CHECK(l0 + (size_t)p.nsplit * s.N * s.Hq * 8 <= ws + need);
                    // the prefix slots (all but the tree's own slot, if any)
                    // cover the longest prefix, and none is empty for it
                    const int npre = p.nsplit - (p.tree_slot ? 1 : 0);
                    CHECK(p.tree_slot == (s.B <= 1 ? 1 : 0));
                    CHECK(p.chunk > 0 && (int64_t)p.chunk * npre >= s.maxpre);
                    CHECK((int64_t)p.chunk * (npre - 1) < s.maxpre);
                }
                CHECK(p.units > 0 && p.units_per_xcd * 8 >= p.units);
                if (need > 0) {
                    // a short or misaligned workspace is refused before any launch
                    const int n0 = ta::n_launch;
                    CHECK(fwd(s, dt, splits, ws, need - 1) == TA_ERR_WORKSPACE);
                    CHECK(fwd(s, dt, splits, ws + 16, need) == TA_ERR_WORKSPACE);
                    CHECK(fwd(s, dt, splits, nullptr, need) == TA_ERR_WORKSPACE);
                    CHECK(ta::n_launch == n0);
                }
            }
        }
        CHECK(tree_attn_num_splits(s.B, s.Hq, s.Hkv, s.D, s.maxt, s.maxpre, TA_DTYPE_BF16) >= 1);
    }
    // invalid shapes and pointers: refused, nothing launched
    const int n0 = ta::n_launch;
    Shape s = shapes[0];
    CHECK(fwd(s, TA_DTYPE_BF16, 0, nullptr, 0, true) == TA_ERR_NULL_PTR ||
          fwd(s, TA_DTYPE_BF16, 0, nullptr, 0, true) == TA_ERR_WORKSPACE);
    Shape t = s; t.D = 96;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_UNSUPPORTED);
    t = s; t.Hq = 30;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_BAD_SHAPE);
    t = s; t.maxt = 257;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_UNSUPPORTED);
    t = s; t.ps = 24;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_UNSUPPORTED);
    t = s; t.maxpre = t.maxp * t.ps + 1;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_BAD_SHAPE);
    t = s; t.N = 17;   // more nodes than B * max_tree
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_BAD_SHAPE);
    CHECK(fwd(s, TA_DTYPE_BF16, 65, nullptr, 0) == TA_ERR_BAD_SHAPE);
    CHECK(fwd(s, (ta_dtype_t)7, 0, nullptr, 0) == TA_ERR_UNSUPPORTED);
    t = s; t.N = 2000000000; t.B = 65535; t.maxt = 256; t.Hq = 32;
    CHECK(fwd(t, TA_DTYPE_BF16, 0, nullptr, 0) == TA_ERR_BAD_SHAPE);
    CHECK(ta::n_launch == n0);
    // sizes from a wide sweep: the pure functions must not overflow
    for (int B = 0; B <= 65535; B = B * 3 + 1)
        for (int maxpre = 0; maxpre <= (1 << 20); maxpre = maxpre * 5 + 1)
            for (int maxt : {0, 1, 16, 64, 65, 256}) {
                (void)tree_attn_num_splits(B, 64, 8, 128, maxt, maxpre, TA_DTYPE_BF16);
                (void)tree_attn_workspace_bytes(B, B * maxt, 64, 8, 128, maxt, maxpre, TA_DTYPE_BF16, 0);
            }
    // the other entry points
    CHECK(tree_attn_plan((const int32_t *)fake(1), (const int32_t *)fake(2), (const int32_t *)fake(3), 4, 100, 64,
                         (uint64_t *)fake(4), (int32_t *)fake(5), (int32_t *)fake(6), (int32_t *)fake(7),
                         nullptr) == TA_OK);
    CHECK(tree_attn_plan(nullptr, (const int32_t *)fake(2), (const int32_t *)fake(3), 4, 100, 64,
                         (uint64_t *)fake(4), (int32_t *)fake(5), (int32_t *)fake(6), (int32_t *)fake(7),
                         nullptr) == TA_ERR_NULL_PTR);
    CHECK(tree_attn_plan((const int32_t *)fake(1), (const int32_t *)fake(2), (const int32_t *)fake(3), 4, 300, 64,
                         (uint64_t *)fake(4), (int32_t *)fake(5), (int32_t *)fake(6), (int32_t *)fake(7),
                         nullptr) == TA_ERR_BAD_SHAPE);
    CHECK(tree_attn_gather_rows(fake(1), 10, (const int32_t *)fake(2), fake(3), 10, 6, nullptr) == TA_ERR_BAD_SHAPE);
    CHECK(tree_attn_gather_rows(fake(1), 10, (const int32_t *)fake(2), fake(3), 10, 64, nullptr) == TA_OK);
    CHECK(tree_attn_build_tree((const float *)fake(1), 32, 16, 8, 256, (int32_t *)fake(2), (int32_t *)fake(3),
                               (float *)fake(4), nullptr) == TA_OK);
    CHECK(tree_attn_build_tree((const float *)fake(1), 32, 2, 2, 256, (int32_t *)fake(2), (int32_t *)fake(3),
                               (float *)fake(4), nullptr) == TA_ERR_BAD_SHAPE);
    CHECK(tree_attn_build_tree((const float *)fake(1), 32, 16, 65, 256, (int32_t *)fake(2), (int32_t *)fake(3),
                               (float *)fake(4), nullptr) == TA_ERR_UNSUPPORTED);
    CHECK(tree_attn_commit((const uint64_t *)fake(1), (const int32_t *)fake(2), (const int32_t *)fake(3),
                           (const int32_t *)fake(4), (const int32_t *)fake(5), fake(6), fake(7), fake(8), fake(9),
                           (const int32_t *)fake(10), 32, 8192, 4, 128, 16, 9000, 260, 256, TA_DTYPE_BF16,
                           (int32_t *)fake(11), (int32_t *)fake(12), nullptr) == TA_OK);
    CHECK(tree_attn_commit((const uint64_t *)fake(1), (const int32_t *)fake(2), (const int32_t *)fake(3),
                           (const int32_t *)fake(4), (const int32_t *)fake(5), fake(6), fake(7), fake(8), fake(9),
                           (const int32_t *)fake(10), 32, 8192, 1, 4, 16, 9000, 260, 256, TA_DTYPE_BF16,
                           (int32_t *)fake(11), (int32_t *)fake(12), nullptr) == TA_ERR_UNSUPPORTED);
    CHECK(strlen(tree_attn_status_str(-42)) > 0 && tree_attn_abi_version() == TREE_ATTN_ABI_VERSION);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host checks ok (%d launches recorded)\n", ta::n_launch);
    return 0;
}
