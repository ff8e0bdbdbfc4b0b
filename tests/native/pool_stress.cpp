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
#include <random>
#include <vector>

#include "../../include/pagedattn.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

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
  std::printf("pool stress ok\n");
  return 0;
}
