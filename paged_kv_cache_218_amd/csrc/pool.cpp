// Host bookkeeping of the paged KV pool: reference counts, the LIFO free list
// and the write plan (allocation on growth, copy-on-write on shared blocks).
//
// The pages fix the behaviour: one block from the free pool per block_size
// tokens of growth, sharers of a prompt point at the same blocks with a count
// equal to the number of sharers, a write into a shared block gives the
// writer a private copy, and a block at count 0 is free again (Blog #54,
// interview question 2; Part 8, "RadixAttention"). Which free block is handed
// out is this library's rule: the free list is a stack whose head is popped
// by an allocation and pushed by a release.
//
// Pure C++ with no HIP dependency, so it is also built and sanitised on the
// host alone.
#include <cstring>
#include <memory>
#include <new>
#include <vector>

#include "pa_internal.h"

extern "C" const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_NO_FREE_BLOCK: return "no free block in the pool";
    case PA_ERR_BAD_BLOCK: return "bad block (free block or refcount underflow)";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_MEMORY: return "out of host memory";
    case PA_ERR_TOO_LARGE: return "needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

extern "C" int64_t pa_pool_buffer_bytes(int32_t num_blocks, int32_t block_size,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (num_blocks <= 0 || num_kv_heads <= 0 || !pa::supported_block_size(block_size) ||
      !pa::supported_head_dim(head_dim))
    return -1;
  const int64_t slots = int64_t(num_blocks) * num_kv_heads * block_size;
  if (dtype == PA_DTYPE_F32 || dtype == PA_DTYPE_BF16) return slots * head_dim * pa::elem_bytes(dtype);
  if (dtype == PA_DTYPE_FP8_E4M3) return slots * head_dim + slots * int64_t(sizeof(float));
  return -1;
}

extern "C" int64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t elem_bytes) {
  if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return -1;
  // one K vector and one V vector per KV head and layer
  return int64_t(2) * num_layers * num_kv_heads * head_dim * elem_bytes;
}

namespace {

pa_status pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, const int32_t* initial_free_order, pa_pool** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_FP8_E4M3)
    return PA_ERR_UNSUPPORTED;
  if (!pa::supported_block_size(block_size) || !pa::supported_head_dim(head_dim))
    return PA_ERR_UNSUPPORTED;
  std::unique_ptr<pa_pool> p(new pa_pool());
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->refcount.assign(num_blocks, 0);
  p->stack.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = initial_free_order ? initial_free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_INVALID_ARG;
    seen[b] = 1;
    // stack top (back) is the head of the free list
    p->stack[num_blocks - 1 - i] = b;
  }
  *out = p.release();
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t dtype,
                                    const int32_t* initial_free_order, pa_pool** out) {
  return pa::guarded([&] {
    return pool_create(num_blocks, block_size, num_kv_heads, head_dim, dtype, initial_free_order, out);
  });
}

// Releasing a pool (and its cache) allocates nothing.
extern "C" void pa_pool_destroy(pa_pool* pool) {
  if (!pool) return;
  if (pool->cache) pa::cache_release(pool->cache);
  delete pool;
}

namespace {

bool in_range(const pa_pool* p, int32_t b) { return b >= 0 && b < p->num_blocks; }

// Whether `need` blocks can be handed out: the free list, then (with a prefix
// cache) the cached blocks eviction can still free.
bool can_supply(const pa_pool* p, int64_t need) {
  int64_t avail = int64_t(p->stack.size());
  if (need > avail && p->cache) avail += pa::cache_reclaimable(p);
  return need <= avail;
}

// Callers check can_supply first.
int32_t pop_free(pa_pool* p) {
  int32_t b;
  if (!p->stack.empty()) {
    b = p->stack.back();
    p->stack.pop_back();
  } else {
    b = pa::cache_evict_one(p);
  }
  p->refcount[b] = 1;
  return b;
}

void release(pa_pool* p, int32_t b) {
  if (--p->refcount[b] == 0) {
    if (p->cache && pa::cache_holds(p, b)) pa::cache_unreferenced(p, b);  // stays cached
    else p->stack.push_back(b);
  }
}

// A write into block b copies it first: other sequences read it, or the
// prefix cache keeps its contents.
bool must_copy(const pa_pool* p, int32_t b) {
  return p->refcount[b] > 1 || (p->cache && pa::cache_holds(p, b));
}

}  // namespace

extern "C" pa_status pa_block_alloc(pa_pool* pool, int32_t* block_id) {
  if (!pool || !block_id) return PA_ERR_INVALID_ARG;
  if (!can_supply(pool, 1)) return PA_ERR_NO_FREE_BLOCK;
  *block_id = pop_free(pool);
  return PA_OK;
}

extern "C" pa_status pa_block_fork(pa_pool* pool, int32_t block_id) {
  if (!pool || !in_range(pool, block_id)) return PA_ERR_INVALID_ARG;
  if (pool->refcount[block_id] == 0) return PA_ERR_BAD_BLOCK;
  ++pool->refcount[block_id];
  return PA_OK;
}

extern "C" pa_status pa_block_free(pa_pool* pool, int32_t block_id) {
  if (!pool || !in_range(pool, block_id)) return PA_ERR_INVALID_ARG;
  if (pool->refcount[block_id] == 0) return PA_ERR_BAD_BLOCK;
  release(pool, block_id);
  return PA_OK;
}

extern "C" pa_status pa_block_refcount(const pa_pool* pool, int32_t block_id, int32_t* refcount) {
  if (!pool || !refcount || !in_range(pool, block_id)) return PA_ERR_INVALID_ARG;
  *refcount = pool->refcount[block_id];
  return PA_OK;
}

extern "C" pa_status pa_pool_num_free(const pa_pool* pool, int32_t* num_free) {
  if (!pool || !num_free) return PA_ERR_INVALID_ARG;
  *num_free = static_cast<int32_t>(pool->stack.size());
  return PA_OK;
}

extern "C" pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t capacity,
                                       int32_t* n) {
  if (!pool || !n) return PA_ERR_INVALID_ARG;
  const int32_t len = static_cast<int32_t>(pool->stack.size());
  *n = len;
  if (!out || capacity < len) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < len; ++i) out[i] = pool->stack[len - 1 - i];
  return PA_OK;
}

namespace pa {

pa_status plan_write(pa_pool* p, int32_t* table, int32_t capacity, int32_t* live_inout,
                     int32_t start_pos, int32_t n_tokens, std::vector<int32_t>* copies,
                     int32_t max_copies, int32_t* slots) {
  if (!p || !table || !live_inout) return PA_ERR_INVALID_ARG;
  const int64_t bs = p->block_size;
  int32_t live = *live_inout;
  if (start_pos < 0 || n_tokens < 0 || live < 0 || live > capacity || capacity < 0)
    return PA_ERR_INVALID_ARG;
  if (copies) copies->clear();
  if (n_tokens == 0) return PA_OK;
  if (int64_t(start_pos) > int64_t(live) * bs) return PA_ERR_INVALID_ARG;  // would leave a hole
  const int64_t end = int64_t(start_pos) + n_tokens;
  const int64_t last_block = (end - 1) / bs;
  if (last_block >= capacity) return PA_ERR_INVALID_ARG;
  const int32_t first_block = static_cast<int32_t>(start_pos / bs);
  const int32_t last = static_cast<int32_t>(last_block);

  // validate and count before changing anything
  int64_t need = last >= live ? int64_t(last) + 1 - live : 0;
  int64_t n_copy = 0;
  for (int32_t j = first_block; j < live && j <= last; ++j) {
    const int32_t b = table[j];
    if (!in_range(p, b)) return PA_ERR_INVALID_ARG;
    if (p->refcount[b] == 0) return PA_ERR_BAD_BLOCK;
    if (must_copy(p, b)) ++n_copy;
  }
  need += n_copy;
  if (copies && n_copy > max_copies) return PA_ERR_INVALID_ARG;
  if (!can_supply(p, need)) return PA_ERR_NO_FREE_BLOCK;
  if (copies) copies->reserve(size_t(2 * n_copy));  // the only allocation, before any change

  for (int32_t j = first_block; j <= last; ++j) {
    if (j < live) {
      const int32_t old = table[j];
      if (must_copy(p, old)) {
        const int32_t fresh = pop_free(p);
        if (copies) {
          copies->push_back(old);
          copies->push_back(fresh);
        }
        release(p, old);
        table[j] = fresh;
      }
    } else {
      table[j] = pop_free(p);
      ++live;
    }
  }
  if (slots) {
    for (int32_t i = 0; i < n_tokens; ++i) {
      const int64_t pos = int64_t(start_pos) + i;
      slots[i] = static_cast<int32_t>(int64_t(table[pos / bs]) * bs + pos % bs);
    }
  }
  *live_inout = live;
  return PA_OK;
}

}  // namespace pa

extern "C" pa_status pa_write_plan(pa_pool* pool, int32_t* block_table, int32_t table_capacity,
                                   int32_t* num_blocks_inout, int32_t start_pos,
                                   int32_t n_tokens, int32_t* copies_out, int32_t max_copies,
                                   int32_t* n_copies_out, int32_t* slots_out) {
  return pa::guarded([&]() -> pa_status {
    std::vector<int32_t> copies;
    const int32_t cap = copies_out ? max_copies : INT32_MAX;
    const pa_status st = pa::plan_write(pool, block_table, table_capacity, num_blocks_inout, start_pos,
                                        n_tokens, &copies, cap, slots_out);
    if (st != PA_OK) return st;
    const int32_t n = static_cast<int32_t>(copies.size() / 2);
    if (n_copies_out) *n_copies_out = n;
    if (copies_out && n) std::memcpy(copies_out, copies.data(), copies.size() * sizeof(int32_t));
    return PA_OK;
  });
}

// Ancestor masks of a tree of drafted tokens: bit j of masks[i] is set when
// node j is node i or one of its ancestors (a candidate token sees the
// candidates it continues; speculative decoding variants, parallel decoding of
// a candidate tree, in "Mở rộng Quy mô và Triển khai", "Giải mã Suy đoán").
extern "C" pa_status pa_tree_masks(const int32_t* parents, int32_t n, uint32_t* masks) {
  if (!parents || !masks || n < 1 || n > PA_TREE_MAX_NODES) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (parents[i] < -1 || parents[i] >= i) return PA_ERR_INVALID_ARG;  // parents come first
  for (int32_t i = 0; i < n; ++i)
    masks[i] = (uint32_t(1) << i) | (parents[i] >= 0 ? masks[parents[i]] : 0u);
  return PA_OK;
}
