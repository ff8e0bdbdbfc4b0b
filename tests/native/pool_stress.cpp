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
// Fault injection: with g_fail_in = k >= 0, k more allocations succeed and
// the next one throws std::bad_alloc (then injection is off again).
static long g_fail_in = -1;
void* operator new(std::size_t n) {
  ++g_news;
  if (g_fail_in == 0) {
    g_fail_in = -1;
    throw std::bad_alloc();
  }
  if (g_fail_in > 0) --g_fail_in;
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

// Every entry point that allocates, made to fail at each of its allocations in
// turn: it must return PA_ERR_NO_MEMORY and leave the pool, the cache and the
// caller's table exactly as they were (and leak nothing: LeakSanitizer runs
// at exit).
struct World {
  pa_pool* pool = nullptr;
  pa_prefix_cache* cache = nullptr;
  std::vector<int32_t> table, toks;
  int32_t live = 0;
};

static const int kFNB = 40, kFBS = 16, kFCAP = 8;

// The same state every time: two requests cached and finished, one request
// holding a matched prefix and its own blocks.
static World make_world() {
  World w;
  CHECK(pa_pool_create(kFNB, kFBS, 2, 64, PA_DTYPE_BF16, nullptr, &w.pool) == PA_OK);
  CHECK(pa_prefix_cache_create(w.pool, &w.cache) == PA_OK);
  for (int r = 0; r < 2; ++r) {
    std::vector<int32_t> toks(kFBS * 3 + 5), tab(kFCAP, -1);
    for (size_t i = 0; i < toks.size(); ++i) toks[i] = int32_t((i * 7 + r * (i >= kFBS ? 1 : 0)) % 5);
    int32_t lv = 0, added = 0;
    CHECK(pa_write_plan(w.pool, tab.data(), kFCAP, &lv, 0, int32_t(toks.size()), nullptr, 0, nullptr, nullptr) == PA_OK);
    CHECK(pa_prefix_insert(w.cache, toks.data(), int32_t(toks.size()), tab.data(), lv, &added) == PA_OK);
    for (int j = 0; j < lv; ++j) CHECK(pa_block_free(w.pool, tab[j]) == PA_OK);
  }
  w.toks.resize(kFBS * 4 + 3);
  for (size_t i = 0; i < w.toks.size(); ++i) w.toks[i] = int32_t((i * 7) % 5);
  w.table.assign(kFCAP, -1);
  int32_t n = 0;
  CHECK(pa_prefix_match(w.cache, w.toks.data(), int32_t(w.toks.size()), w.table.data(), kFCAP, &n) == PA_OK);
  w.live = n;
  CHECK(pa_write_plan(w.pool, w.table.data(), kFCAP, &w.live, n * kFBS, int32_t(w.toks.size()) - n * kFBS,
                      nullptr, 0, nullptr, nullptr) == PA_OK);
  return w;
}

struct Snapshot {
  std::vector<int32_t> rc, fl, blocks, parents, table;
  std::vector<int64_t> stamps;
  int32_t live = 0;
  bool operator==(const Snapshot& o) const {
    return rc == o.rc && fl == o.fl && blocks == o.blocks && parents == o.parents && stamps == o.stamps &&
           table == o.table && live == o.live;
  }
};

static Snapshot snap(const World& w) {
  Snapshot s;
  s.rc.assign(kFNB, 0);
  for (int b = 0; b < kFNB; ++b) CHECK(pa_block_refcount(w.pool, b, &s.rc[b]) == PA_OK);
  int32_t n = 0;
  s.fl.assign(kFNB, -1);
  CHECK(pa_pool_free_list(w.pool, s.fl.data(), kFNB, &n) == PA_OK);
  s.fl.resize(n);
  s.blocks.assign(kFNB, 0);
  s.parents.assign(kFNB, 0);
  s.stamps.assign(kFNB, 0);
  CHECK(pa_prefix_cache_dump(w.cache, s.blocks.data(), s.parents.data(), s.stamps.data(), kFNB, &n) == PA_OK);
  s.blocks.resize(n);
  s.parents.resize(n);
  s.stamps.resize(n);
  s.table = w.table;
  s.live = w.live;
  return s;
}

static void fault_injection() {
  // each call, run on a fresh copy of the same state with the k-th allocation failing
  auto probe = [](const char* what, auto call) {
    for (long k = 0;; ++k) {
      World w = make_world();
      const Snapshot before = snap(w);
      const pa_status st = call(w, k);  // arms the injection right before the call under test
      const bool injected = g_fail_in == -1;
      g_fail_in = -1;
      if (injected) {
        if (st != PA_ERR_NO_MEMORY || !(snap(w) == before)) {
          std::fprintf(stderr, "%s: allocation %ld failing gave status %d or changed the state\n", what, k, st);
          std::exit(1);
        }
      } else {
        CHECK(st == PA_OK);  // needed at most k allocations: the call ran to the end
        CHECK(k > 0);        // and it did allocate, so the failures were exercised
        std::printf("%s: each of %ld allocations failing left the state unchanged\n", what, k);
        pa_pool_destroy(w.pool);
        break;
      }
      pa_pool_destroy(w.pool);
      CHECK(k < 10000);
    }
  };
  probe("pa_write_plan (rewrite of cached blocks)", [](World& w, long k) {
    std::vector<int32_t> copies(2 * kFCAP);
    int32_t ncp = 0;
    g_fail_in = k;
    return pa_write_plan(w.pool, w.table.data(), kFCAP, &w.live, 0, 2 * kFBS, copies.data(), kFCAP, &ncp, nullptr);
  });
  probe("pa_prefix_match", [](World& w, long k) {
    std::vector<int32_t> t(kFCAP, -1);
    int32_t n = 0;
    g_fail_in = k;
    return pa_prefix_match(w.cache, w.toks.data(), int32_t(w.toks.size()), t.data(), kFCAP, &n);
  });
  probe("pa_prefix_insert", [](World& w, long k) {
    int32_t added = 0;
    g_fail_in = k;
    return pa_prefix_insert(w.cache, w.toks.data(), int32_t(w.toks.size()), w.table.data(), w.live, &added);
  });
  probe("pa_pool_create", [](World&, long k) {
    pa_pool* p = nullptr;
    g_fail_in = k;
    const pa_status st = pa_pool_create(kFNB, kFBS, 2, 64, PA_DTYPE_BF16, nullptr, &p);
    const long left = g_fail_in;
    g_fail_in = -1;
    CHECK((st == PA_OK) == (p != nullptr));
    if (p) pa_pool_destroy(p);
    g_fail_in = left;
    return st;
  });
  probe("pa_prefix_cache_create", [](World&, long k) {
    pa_pool* p = nullptr;
    CHECK(pa_pool_create(kFNB, kFBS, 2, 64, PA_DTYPE_BF16, nullptr, &p) == PA_OK);
    pa_prefix_cache* c = nullptr;
    g_fail_in = k;
    const pa_status st = pa_prefix_cache_create(p, &c);
    const long left = g_fail_in;
    g_fail_in = -1;
    CHECK((st == PA_OK) == (c != nullptr));
    pa_pool_destroy(p);
    g_fail_in = left;
    return st;
  });
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
  fault_injection();
  std::printf("pool stress ok\n");
  return 0;
}
