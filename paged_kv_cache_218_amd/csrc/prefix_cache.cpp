// Radix-tree prefix cache over the block pool (host bookkeeping).
//
// Part 8, "RadixAttention": KV blocks of earlier requests are kept in a
// prefix tree; a request whose tokens match a cached prefix reuses those
// physical blocks by incrementing their reference counts (and skips their
// prefill); under memory pressure an LRU policy frees blocks whose count is 0.
// "Mở rộng Quy mô và Triển khai", "Cache Tiền tố": the longest cached prefix
// is found and generation starts from there.
//
// The mechanics, which the pages leave open, are this library's: one tree
// node per full block keyed by its block_size token ids; a cached block whose
// count falls to 0 stays in the tree, stamped with a counter, instead of
// returning to the free list; when the free list is empty, allocation evicts
// the unreferenced leaf with the oldest stamp (leaves only, so every cached
// block stays reachable); a block is reclaimable when it and its whole
// subtree are unreferenced; a write into a cached block copies it first.
//
// Pure C++, no HIP: built and sanitised on the host alone.
#include <algorithm>
#include <map>
#include <memory>
#include <new>
#include <set>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace {

// Blocks ordered by (stamp, block id): an indexed binary min-heap with room
// for every block of the pool, allocated with the cache, so that the pool
// operations that reach it (a release, an allocation that evicts) never
// allocate. The stamps of the blocks it holds do not change while they are in.
class BlockHeap {
 public:
  void init(size_t num_blocks, const std::vector<int64_t>* stamps) {
    heap_.assign(num_blocks, -1);
    pos_.assign(num_blocks, -1);
    size_ = 0;
    stamp_ = stamps;
  }
  bool empty() const { return size_ == 0; }
  int32_t top() const { return size_ > 0 ? heap_[0] : -1; }
  void insert(int32_t b) {
    if (pos_[b] >= 0) return;
    heap_[size_] = b;
    pos_[b] = size_;
    up(size_++);
  }
  void erase(int32_t b) {
    const int32_t i = pos_[b];
    if (i < 0) return;
    pos_[b] = -1;
    if (i == --size_) return;
    const int32_t moved = heap_[size_];
    heap_[i] = moved;
    pos_[moved] = i;
    up(i);
    down(pos_[moved]);
  }

 private:
  bool before(int32_t a, int32_t b) const {
    const int64_t sa = (*stamp_)[a], sb = (*stamp_)[b];
    return sa < sb || (sa == sb && a < b);
  }
  void swap_at(int32_t i, int32_t j) {
    std::swap(heap_[i], heap_[j]);
    pos_[heap_[i]] = i;
    pos_[heap_[j]] = j;
  }
  void up(int32_t i) {
    while (i > 0) {
      const int32_t par = (i - 1) / 2;
      if (!before(heap_[i], heap_[par])) break;
      swap_at(i, par);
      i = par;
    }
  }
  void down(int32_t i) {
    for (;;) {
      const int32_t l = 2 * i + 1, r = l + 1;
      int32_t m = i;
      if (l < size_ && before(heap_[l], heap_[m])) m = l;
      if (r < size_ && before(heap_[r], heap_[m])) m = r;
      if (m == i) return;
      swap_at(i, m);
      i = m;
    }
  }
  std::vector<int32_t> heap_, pos_;
  int32_t size_ = 0;
  const std::vector<int64_t>* stamp_ = nullptr;
};

}  // namespace

struct pa_prefix_cache {
  pa_pool* pool = nullptr;
  int64_t clock = 0;                      // bumped each time a cached block becomes unreferenced
  std::vector<char> cached;               // per block: in the tree
  std::vector<int32_t> parent;            // per block: parent block, -1 for a child of the root
  std::vector<std::vector<int32_t>> key;  // per block: its block_size token ids
  std::vector<std::map<std::vector<int32_t>, int32_t>> children;  // per block
  std::map<std::vector<int32_t>, int32_t> roots;                  // children of the root
  std::vector<int64_t> stamp;             // per block: when it became unreferenced, or -1
  BlockHeap leaves;                       // unreferenced leaves by (stamp, block)
  // scratch of cache_reclaimable, sized for every block when the cache is made
  std::vector<int32_t> walk_order, walk_stack;
  std::vector<char> walk_live;
};

namespace {

std::map<std::vector<int32_t>, int32_t>& children_of(pa_prefix_cache* c, int32_t node) {
  return node < 0 ? c->roots : c->children[node];
}

// Take block b (an unreferenced leaf) out of the tree.
void detach(pa_prefix_cache* c, int32_t b) {
  c->leaves.erase(b);
  const int32_t par = c->parent[b];
  children_of(c, par).erase(c->key[b]);
  c->cached[b] = 0;
  c->parent[b] = -1;
  c->key[b].clear();
  c->stamp[b] = -1;
  if (par >= 0 && c->stamp[par] >= 0 && c->children[par].empty()) c->leaves.insert(par);
}

int32_t evict_one(pa_prefix_cache* c) {
  if (c->leaves.empty()) return -1;
  const int32_t b = c->leaves.top();
  detach(c, b);
  return b;
}

}  // namespace

namespace pa {

bool cache_holds(const pa_pool* p, int32_t b) { return p->cache->cached[b] != 0; }

void cache_unreferenced(pa_pool* p, int32_t b) {
  pa_prefix_cache* c = p->cache;
  c->stamp[b] = ++c->clock;
  if (c->children[b].empty()) c->leaves.insert(b);
}

// Unreferenced blocks with no referenced block below them: children are
// visited before their parents (iterative, the tree can be deep).
// No allocation: the walk uses the cache's preallocated scratch (each cached
// block enters the stack and the order once).
int64_t cache_reclaimable(const pa_pool* p) {
  pa_prefix_cache* c = p->cache;
  std::vector<int32_t>& order = c->walk_order;
  std::vector<int32_t>& stack = c->walk_stack;
  std::vector<char>& live = c->walk_live;
  order.clear();
  stack.clear();
  for (const auto& kv : c->roots) stack.push_back(kv.second);
  while (!stack.empty()) {
    const int32_t n = stack.back();
    stack.pop_back();
    order.push_back(n);
    for (const auto& kv : c->children[n]) stack.push_back(kv.second);
  }
  std::fill(live.begin(), live.end(), 0);
  int64_t count = 0;
  for (auto it = order.rbegin(); it != order.rend(); ++it) {
    const int32_t n = *it;
    bool l = p->refcount[n] > 0;
    for (const auto& kv : c->children[n]) l = l || live[kv.second];
    live[n] = l;
    if (!l) ++count;
  }
  return count;
}

int32_t cache_evict_one(pa_pool* p) { return evict_one(p->cache); }

void cache_release(pa_prefix_cache* c) {
  pa_pool* p = c->pool;
  // reclaimable blocks to the free list in eviction order, then any other
  // unreferenced cached block (ascending stamp); referenced ones go back to
  // the free list when their holders release them
  for (int32_t b = evict_one(c); b >= 0; b = evict_one(c)) p->stack.push_back(b);
  for (int32_t b = 0; b < p->num_blocks; ++b)
    if (c->cached[b] && c->stamp[b] >= 0) c->leaves.insert(b);
  for (int32_t b = c->leaves.top(); b >= 0; b = c->leaves.top()) {
    c->leaves.erase(b);
    p->stack.push_back(b);
  }
  p->cache = nullptr;
  delete c;
}

}  // namespace pa

extern "C" pa_status pa_prefix_cache_create(pa_pool* pool, pa_prefix_cache** out) {
  if (!pool || !out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (pool->cache) return PA_ERR_INVALID_ARG;  // one cache per pool
  return pa::guarded([&]() -> pa_status {
    std::unique_ptr<pa_prefix_cache> c(new pa_prefix_cache());
    const size_t nb = size_t(pool->num_blocks);
    c->pool = pool;
    c->cached.assign(nb, 0);
    c->parent.assign(nb, -1);
    c->key.assign(nb, {});
    c->children.assign(nb, {});
    c->stamp.assign(nb, -1);
    c->leaves.init(nb, &c->stamp);
    c->walk_order.reserve(nb);
    c->walk_stack.reserve(nb);
    c->walk_live.assign(nb, 0);
    pool->cache = c.get();
    *out = c.release();
    return PA_OK;
  });
}

extern "C" void pa_prefix_cache_destroy(pa_prefix_cache* cache) {
  if (cache) pa::cache_release(cache);
}

extern "C" pa_status pa_prefix_match(pa_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                                     int32_t* table, int32_t capacity, int32_t* n_blocks) {
  if (!cache || !n_blocks || n_tokens < 0 || capacity < 0 || (n_tokens > 0 && !tokens) ||
      (capacity > 0 && !table))
    return PA_ERR_INVALID_ARG;
  return pa::guarded([&]() -> pa_status {
    pa_pool* p = cache->pool;
    const int32_t bs = p->block_size;
    std::vector<int32_t> chunk(bs);  // the only allocation, before any change
    int32_t node = -1, n = 0;
    const int32_t most = std::min(n_tokens / bs, capacity);
    for (; n < most; ++n) {
      chunk.assign(tokens + int64_t(n) * bs, tokens + int64_t(n + 1) * bs);
      auto& kids = children_of(cache, node);
      const auto it = kids.find(chunk);
      if (it == kids.end()) break;
      node = it->second;
      table[n] = node;
    }
    for (int32_t i = 0; i < n; ++i) {  // fork the matched blocks, reviving unreferenced ones
      const int32_t b = table[i];
      if (p->refcount[b] == 0) {
        cache->leaves.erase(b);
        cache->stamp[b] = -1;
      }
      ++p->refcount[b];
    }
    *n_blocks = n;
    return PA_OK;
  });
}

extern "C" pa_status pa_prefix_insert(pa_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                                      const int32_t* table, int32_t n_blocks, int32_t* n_new) {
  if (!cache || n_tokens < 0 || n_blocks < 0 || (n_tokens > 0 && !tokens) || (n_blocks > 0 && !table))
    return PA_ERR_INVALID_ARG;
  return pa::guarded([&]() -> pa_status {
    pa_pool* p = cache->pool;
    const int32_t bs = p->block_size;
    const int32_t n = std::min(n_blocks, n_tokens / bs);
    // Everything the insertion needs is allocated while planning (the tree
    // node, with its key, and the block's own copy of the key), so that
    // applying the plan allocates nothing and cannot stop half way.
    using Children = std::map<std::vector<int32_t>, int32_t>;
    struct Planned {
      int32_t parent;
      Children::node_type node;
      std::vector<int32_t> key;
      int32_t block;
    };
    std::vector<Planned> plan;
    plan.reserve(size_t(n));
    std::set<int32_t> planned;
    int32_t node = -1;
    bool fresh = false;  // below a planned node: nothing cached yet
    for (int32_t i = 0; i < n; ++i) {
      std::vector<int32_t> chunk(tokens + int64_t(i) * bs, tokens + int64_t(i + 1) * bs);
      int32_t child = -1;
      if (!fresh) {
        auto& kids = children_of(cache, node);
        const auto it = kids.find(chunk);
        if (it != kids.end()) child = it->second;
      }
      if (child >= 0) {
        node = child;
        continue;
      }
      const int32_t b = table[i];
      if (b < 0 || b >= p->num_blocks) return PA_ERR_INVALID_ARG;
      if (p->refcount[b] == 0) return PA_ERR_BAD_BLOCK;
      if (cache->cached[b] || planned.count(b)) return PA_ERR_INVALID_ARG;  // cached under another prefix
      Children holder;
      holder.emplace(chunk, b);
      plan.push_back({node, holder.extract(holder.begin()), std::move(chunk), b});
      planned.insert(b);
      node = b;
      fresh = true;
    }
    for (auto& pl : plan) {
      if (pl.parent >= 0 && cache->stamp[pl.parent] >= 0 && cache->children[pl.parent].empty())
        cache->leaves.erase(pl.parent);  // no longer a leaf
      cache->cached[pl.block] = 1;
      cache->parent[pl.block] = pl.parent;
      cache->key[pl.block] = std::move(pl.key);
      cache->stamp[pl.block] = -1;
      children_of(cache, pl.parent).insert(std::move(pl.node));
    }
    if (n_new) *n_new = int32_t(plan.size());
    return PA_OK;
  });
}

extern "C" pa_status pa_prefix_evict(pa_prefix_cache* cache, int32_t max_blocks, int32_t* evicted,
                                     int32_t* n_evicted) {
  if (!cache || max_blocks < 0 || !n_evicted) return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  while (n < max_blocks) {
    const int32_t b = evict_one(cache);
    if (b < 0) break;
    cache->pool->stack.push_back(b);
    if (evicted) evicted[n] = b;
    ++n;
  }
  *n_evicted = n;
  return PA_OK;
}

extern "C" pa_status pa_prefix_cache_stats(const pa_prefix_cache* cache, int32_t* cached,
                                           int32_t* unreferenced, int32_t* reclaimable) {
  if (!cache) return PA_ERR_INVALID_ARG;
  int32_t nc = 0, nu = 0;
  for (size_t b = 0; b < cache->cached.size(); ++b) {
    nc += cache->cached[b] ? 1 : 0;
    nu += (cache->cached[b] && cache->stamp[b] >= 0) ? 1 : 0;
  }
  if (cached) *cached = nc;
  if (unreferenced) *unreferenced = nu;
  if (reclaimable) *reclaimable = int32_t(pa::cache_reclaimable(cache->pool));
  return PA_OK;
}

extern "C" pa_status pa_prefix_cache_dump(const pa_prefix_cache* cache, int32_t* blocks, int32_t* parents,
                                          int64_t* stamps, int32_t capacity, int32_t* n) {
  if (!cache || !n) return PA_ERR_INVALID_ARG;
  int32_t k = 0;
  for (size_t b = 0; b < cache->cached.size(); ++b)
    if (cache->cached[b]) ++k;
  *n = k;
  if (!blocks || !parents || !stamps || capacity < k) return PA_ERR_INVALID_ARG;
  k = 0;
  for (size_t b = 0; b < cache->cached.size(); ++b) {
    if (!cache->cached[b]) continue;
    blocks[k] = int32_t(b);
    parents[k] = cache->parent[b];
    stamps[k] = cache->stamp[b];
    ++k;
  }
  return PA_OK;
}
