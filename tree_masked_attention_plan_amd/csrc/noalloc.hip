// tree_attn_fwd_noalloc: tree_attn_fwd with the split workspace taken from a
// fixed device array instead of the caller, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The array lives for the whole process on every device the library runs on;
// its device address is looked up once per device (with that device current)
// and kept.  Host code never uses the array's name as an address: in host
// code that name is only a stand-in, and the kernels get the looked-up
// pointer, as they get a caller's workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tree_attn.h"

namespace {

// the largest split workspace this entry point serves (bytes)
constexpr size_t kScratchBytes = (size_t)TREE_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices];   // looked-up address of scratch on each device

// The device address of this device's copy of scratch (nullptr on failure).
void *scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

ta_status_t tree_attn_fwd_noalloc(const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                                  const void *v_cache, const int32_t *block_table, const int32_t *prefix_len,
                                  const int32_t *tree_off, const uint64_t *anc_mask, int32_t B, int32_t N,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                  int32_t max_pages_per_seq, int32_t max_tree, int32_t max_prefix,
                                  float softmax_scale, ta_dtype_t dtype, int32_t num_splits, void *out,
                                  float *lse, void *stream)
{
    const size_t need = tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_tree, max_prefix, dtype, num_splits);
    if (need > kScratchBytes)
        return TA_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (ws == nullptr)
            return TA_ERR_HIP;
    }
    return tree_attn_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask, B, N,
                         Hq, Hkv, D, page_size, num_pages, max_pages_per_seq, max_tree, max_prefix, softmax_scale,
                         dtype, num_splits, out, lse, ws, need, stream);
}

}  // extern "C"
