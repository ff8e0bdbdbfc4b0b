// Host-only stress of the pool bookkeeping (pool.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_native_sanitizers.py.
// Random alloc / fork / free / write-plan operations, with the pool's
// invariants checked after every step:
//   * every block is either free (count 0, exactly once in the free list) or
//     live (count > 0, not in the free list);
//   * the counts equal the number of table entries naming each block plus the
//     extra references this driver holds;
//   * errors leave the pool unchanged.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <random>
#include <vector>

#include "../../include/pagedattn.h"

// Every operator new of the program is counted, so that the pool and cache
// operations that must not allocate (a release, an allocation, an eviction,
// the statistics, destroying the pool) can be checked to allocate nothing.
static long g_news = 0;
void* operator new(std::size_t n) {
  ++g_news;
  if (void* p = std::malloc(n ? n : 1)) return p;
  throw std::bad_alloc();
}
void* operator new[](std::size_t n) { return operator new(n); }
void operator delete(void* p) noexcept { std::free(p); }
void operator delete[](void* p) noexcept { std::free(p); }
void operator delete(void* p, std::size_t) noexcept { std::free(p); }
void operator delete[](void* p, std::size_t) noexcept { std::free(p); }

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

// expr runs without a single operator new
#define NO_ALLOC(expr)            \
  do {                            \
    const long news0 = g_news;    \
    expr;                         \
    CHECK(g_news == news0);       \
  } while (0)

// Requests sharing a few prompts against a pool with a prefix cache: match,
// write, insert, rewrite, finish and evict at random; the sum of the tables'
// holdings must equal the refcounts, and free + cached + held must cover the
// pool. Destroying the pool with the cache attached must free everything.
static void prefix_cache_stress() {
  const int NB = 96, BS = 16, CAP = 10, NSEQ = 12;
  std::mt19937 rng(7);
  pa_pool* pool = nullptr;
  CHECK(pa_pool_create(NB, BS, 2, 64, PA_DTYPE_BF16, nullptr, &pool) == PA_OK);
  pa_prefix_cache* cache = nullptr;
  const long news_before_cache = g_news;
  CHECK(pa_prefix_cache_create(pool, &cache) == PA_OK);
  CHECK(g_news > news_before_cache);  // the counting operator new is the one in use
  std::vector<std::vector<int32_t>> prompts(4);
  for (auto& pr : prompts) {
    pr.resize(BS * (1 + rng() % 5) + rng() % BS);
    for (auto& t : pr) t = int32_t(rng() % 3);
  }
  std::vector<std::vector<int32_t>> tables(NSEQ, std::vector<int32_t>(CAP, -1)), toks(NSEQ);
  std::vector<int32_t> live(NSEQ, 0);
  for (int step = 0; step < 20000; ++step) {
    const int s = int(rng() % NSEQ), op = int(rng() % 6);
    if (live[s] == 0) {  // start a request
      toks[s] = prompts[rng() % prompts.size()];
      for (int k = int(rng() % BS); k > 0; --k) toks[s].push_back(int32_t(rng() % 3));
      if (int(toks[s].size()) > CAP * BS) toks[s].resize(CAP * BS);
      int32_t n = 0;
      CHECK(pa_prefix_match(cache, toks[s].data(), int32_t(toks[s].size()), tables[s].data(), CAP, &n) == PA_OK);
      int32_t lv = n;
      const pa_status st = pa_write_plan(pool, tables[s].data(), CAP, &lv, n * BS,
                                         int32_t(toks[s].size()) - n * BS, nullptr, 0, nullptr, nullptr);
      if (st == PA_OK) {
        live[s] = lv;
      } else {
        CHECK(st == PA_ERR_NO_FREE_BLOCK);
        for (int j = 0; j < n; ++j) CHECK(pa_block_free(pool, tables[s][j]) == PA_OK);
        tables[s].assign(CAP, -1);
      }
    } else if (op == 0) {
      int32_t added = 0;
      const pa_status st = pa_prefix_insert(cache, toks[s].data(), int32_t(toks[s].size()), tables[s].data(),
                                            live[s], &added);
      CHECK(st == PA_OK || st == PA_ERR_INVALID_ARG);
    } else if (op == 1) {  // rewrite one position
      int32_t lv = live[s];
      const int32_t pos = int32_t(rng() % (live[s] * BS));
      const pa_status st = pa_write_plan(pool, tables[s].data(), CAP, &lv, pos, 1, nullptr, 0, nullptr, nullptr);
      CHECK(st == PA_OK || st == PA_ERR_NO_FREE_BLOCK);
    } else if (op == 2) {
      int32_t ev[8], n = 0;
      NO_ALLOC(CHECK(pa_prefix_evict(cache, int32_t(rng() % 8), ev, &n) == PA_OK));
    } else if (op == 3) {  // a block taken and given back: may evict, never allocates
      int32_t b = -1;
      pa_status st = PA_OK;
      NO_ALLOC(st = pa_block_alloc(pool, &b));
      CHECK(st == PA_OK || st == PA_ERR_NO_FREE_BLOCK);
      if (st == PA_OK) NO_ALLOC(CHECK(pa_block_free(pool, b) == PA_OK));
    } else {  // finish
      for (int j = 0; j < live[s]; ++j) NO_ALLOC(CHECK(pa_block_free(pool, tables[s][j]) == PA_OK));
      tables[s].assign(CAP, -1);
      live[s] = 0;
    }
    if (step % 53 == 0) {
      std::vector<int32_t> held(NB, 0);
      for (int q = 0; q < NSEQ; ++q)
        for (int j = 0; j < live[q]; ++j) ++held[tables[q][j]];
      int32_t nfree = 0, cached = 0, unref = 0, recl = 0;
      CHECK(pa_pool_num_free(pool, &nfree) == PA_OK);
      NO_ALLOC(CHECK(pa_prefix_cache_stats(cache, &cached, &unref, &recl) == PA_OK));
      int referenced = 0;
      for (int b = 0; b < NB; ++b) {
        int32_t rc = -1;
        CHECK(pa_block_refcount(pool, b, &rc) == PA_OK);
        CHECK(rc == held[b]);
        referenced += rc > 0;
      }
      CHECK(nfree + unref + referenced == NB && recl <= unref);
    }
  }
  NO_ALLOC(pa_pool_destroy(pool));  // also destroys the attached cache
}

int main() {
  const int NB = 96, BS = 16, CAP = 24, NSEQ = 8;
  std::mt19937 rng(218);
  std::vector<int32_t> order(NB);
  for (int i = 0; i < NB; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pa_pool* pool = nullptr;
  CHECK(pa_pool_create(NB, BS, 2, 64, PA_DTYPE_BF16, order.data(), &pool) == PA_OK);
  std::vector<std::vector<int32_t>> tables(NSEQ, std::vector<int32_t>(CAP, -1));
  std::vector<int32_t> live(NSEQ, 0), len(NSEQ, 0);
  std::vector<int32_t> extra;  // references held by the driver itself
  auto snapshot = [&](std::vector<int32_t>& rc, std::vector<int32_t>& fl) {
    rc.assign(NB, 0);
    for (int b = 0; b < NB; ++b) CHECK(pa_block_refcount(pool, b, &rc[b]) == PA_OK);
    int32_t n = 0;
    fl.assign(NB, -1);
    CHECK(pa_pool_free_list(pool, fl.data(), NB, &n) == PA_OK);
    fl.resize(n);
  };
  auto check_invariants = [&]() {
    std::vector<int32_t> rc, fl;
    snapshot(rc, fl);
    std::vector<int> want(NB, 0), in_free(NB, 0);
    for (int s = 0; s < NSEQ; ++s)
      for (int j = 0; j < live[s]; ++j) ++want[tables[s][j]];
    for (int32_t b : extra) ++want[b];
    for (int32_t b : fl) {
      CHECK(b >= 0 && b < NB);
      ++in_free[b];
    }
    for (int b = 0; b < NB; ++b) {
      CHECK(rc[b] == want[b]);
      CHECK(in_free[b] == (rc[b] == 0 ? 1 : 0));
    }
  };
  std::vector<int32_t> copies(2 * CAP), slots(CAP * BS);
  for (int step = 0; step < 20000; ++step) {
    const int s = int(rng() % NSEQ);
    const int op = int(rng() % 10);
    std::vector<int32_t> rc0, fl0;
    snapshot(rc0, fl0);
    if (op < 5) {  // write tokens (append or overwrite)
      const int start = len[s] > 0 ? int(rng() % (len[s] + 1)) : 0;
      const int n = 1 + int(rng() % 40);
      std::vector<int32_t> t0 = tables[s];
      int32_t lv = live[s], ncp = 0;
      const pa_status st = pa_write_plan(pool, tables[s].data(), CAP, &lv, start, n, copies.data(),
                                         CAP, &ncp, slots.data());
      if (st == PA_OK) {
        live[s] = lv;
        if (start + n > len[s]) len[s] = start + n;
        for (int i = 0; i < n; ++i) {
          const int p = start + i;
          CHECK(slots[i] == tables[s][p / BS] * BS + p % BS);
        }
      } else {
        CHECK(st == PA_ERR_NO_FREE_BLOCK || st == PA_ERR_INVALID_ARG);
        CHECK(tables[s] == t0);
        std::vector<int32_t> rc1, fl1;
        snapshot(rc1, fl1);
        CHECK(rc1 == rc0 && fl1 == fl0);
      }
    } else if (op < 7) {  // another sequence adopts this one's blocks
      const int d = int(rng() % NSEQ);
      if (d == s) continue;
      for (int j = 0; j < live[d]; ++j) CHECK(pa_block_free(pool, tables[d][j]) == PA_OK);
      for (int j = 0; j < live[s]; ++j) CHECK(pa_block_fork(pool, tables[s][j]) == PA_OK);
      tables[d] = tables[s];
      live[d] = live[s];
      len[d] = len[s];
    } else if (op < 8) {  // the driver takes or drops an extra reference
      if (!extra.empty() && (rng() & 1)) {
        CHECK(pa_block_free(pool, extra.back()) == PA_OK);
        extra.pop_back();
      } else {
        int32_t b = -1;
        const pa_status st = pa_block_alloc(pool, &b);
        if (st == PA_OK) extra.push_back(b);
        else CHECK(st == PA_ERR_NO_FREE_BLOCK);
      }
    } else {  // the sequence finishes
      for (int j = 0; j < live[s]; ++j) CHECK(pa_block_free(pool, tables[s][j]) == PA_OK);
      tables[s].assign(CAP, -1);
      live[s] = len[s] = 0;
    }
    // misuse must fail without changing anything
    if (step % 17 == 0) {
      std::vector<int32_t> rc1, fl1;
      snapshot(rc1, fl1);
      if (!fl1.empty()) {
        CHECK(pa_block_free(pool, fl1[0]) == PA_ERR_BAD_BLOCK);
        CHECK(pa_block_fork(pool, fl1[0]) == PA_ERR_BAD_BLOCK);
      }
      CHECK(pa_block_free(pool, NB) == PA_ERR_INVALID_ARG);
      CHECK(pa_block_fork(pool, -1) == PA_ERR_INVALID_ARG);
      std::vector<int32_t> rc2, fl2;
      snapshot(rc2, fl2);
      CHECK(rc1 == rc2 && fl1 == fl2);
    }
    check_invariants();
  }
  pa_pool_destroy(pool);
  prefix_cache_stress();
  std::printf("pool stress ok\n");
  return 0;
}
