// Internal declarations shared by the host bookkeeping and the HIP launch code.
#pragma once

#include <cstdint>
#include <climits>
#include <new>
#include <vector>

#include "../../include/pagedattn.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t dtype = 0;
  std::vector<int32_t> refcount;  // per physical block
  std::vector<int32_t> stack;     // free list; back() is the head
  pa_prefix_cache* cache = nullptr;  // attached prefix cache, if any
};

namespace pa {

inline bool supported_block_size(int32_t bs) { return bs == 16 || bs == 32; }
inline bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }
inline int32_t elem_bytes(int32_t dtype) {
  return dtype == PA_DTYPE_F32 ? 4 : (dtype == PA_DTYPE_BF16 ? 2 : 1);
}
// Bytes of the codes part of an FP8 pool buffer (the scales follow).
inline int64_t fp8_codes_bytes(int64_t num_blocks, int64_t hkv, int64_t bs, int64_t d) {
  return num_blocks * hkv * bs * d;
}

// Prefix-cache hooks used by the pool (defined with the cache).
bool cache_holds(const pa_pool* p, int32_t block);       // block is in the tree
void cache_unreferenced(pa_pool* p, int32_t block);      // a cached block's count fell to 0
int64_t cache_reclaimable(const pa_pool* p);             // blocks eviction can still free
int32_t cache_evict_one(pa_pool* p);                     // LRU unreferenced leaf, or -1
void cache_release(pa_prefix_cache* c);                  // detach from the pool and delete

// Run `body` (which returns a pa_status) so that no C++ exception crosses the
// C interface: the only ones the standard containers used here throw are
// allocation failures (bad_alloc, length_error), reported as
// PA_ERR_NO_MEMORY. Every entry point that allocates does so before it
// changes any state, so such a failure leaves the handle as it was.
template <typename F>
pa_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
}

// Record a failed HIP call (this thread's last one, read by pa_last_hip_error)
// and return PA_ERR_HIP. Defined with the HIP sources.
pa_status hip_failed(int hip_error);

// Host planning of a write (allocation on growth, copy-on-write on shared
// blocks). copies receives (src, dst) pairs; slots may be null.
pa_status plan_write(pa_pool* p, int32_t* table, int32_t capacity, int32_t* live_inout,
                     int32_t start_pos, int32_t n_tokens, std::vector<int32_t>* copies,
                     int32_t max_copies, int32_t* slots);

}  // namespace pa
