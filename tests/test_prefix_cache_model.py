"""Pins of the radix prefix cache model (CPU only): the pages' narrative
(Part 8, "RadixAttention"), and invariants checked by brute force after
every operation of random request streams."""
import copy

import numpy as np
import pytest

from oracle.allocator import ERR_INVALID_ARG, ERR_NO_FREE_BLOCK, PoolError
from oracle.prefix_cache import PrefixCachedPool

BS = 4


def write_seq(pool, tokens, cap=16, table=None, live=0, start=0):
    table = [-1] * cap if table is None else table
    live, _ = pool.plan_write(table, cap, live, start, len(tokens) - start)
    return table, live


def test_shared_system_prompt_is_matched_and_prefill_skipped():
    pool = PrefixCachedPool(32, BS)
    prompt = list(range(100, 113))                       # 3 full blocks + 1 token
    a, la = write_seq(pool, prompt + [7, 8])             # request A: prompt + reply
    assert pool.insert(prompt + [7, 8], a, la) == 3      # full blocks 0..2 (block 3 is partial)
    for j in range(la):
        pool.free(a[j])
    # the cached blocks stay out of the free list, unreferenced
    assert sorted(b for b, _, t in pool.dump() if t > 0) == sorted(a[:3])
    assert all(b not in pool.free_list() for b in a[:3]) and a[3] in pool.free_list()
    # request B shares the prompt: its first 3 blocks come from the cache
    b = [-1] * 16
    m = pool.match(prompt + [9, 9, 9], 16)
    assert m == a[:3] and all(pool.refcount[x] == 1 for x in m)
    b[:3] = m
    b, lb = write_seq(pool, prompt + [9, 9, 9], table=b, live=3, start=12)   # skips 12 tokens of prefill
    assert b[:3] == a[:3] and lb == 4
    # a third request forks the same blocks: counts 2 (the pages' ref_count++)
    c = pool.match(prompt, 16)
    assert c == a[:3] and all(pool.refcount[x] == 2 for x in c)


def test_lru_evicts_oldest_unreferenced_leaf_first():
    pool = PrefixCachedPool(6, BS, initial_free_order=range(6))
    s1, l1 = write_seq(pool, list(range(8)))              # blocks 0, 1
    pool.insert(list(range(8)), s1, l1)
    s2, l2 = write_seq(pool, [50 + t for t in range(8)])  # blocks 2, 3
    pool.insert([50 + t for t in range(8)], s2, l2)
    for j in (0, 1):
        pool.free(s2[j])                                  # stamps 1 (block 2), 2 (block 3)
    for j in (0, 1):
        pool.free(s1[j])                                  # stamps 3 (block 0), 4 (block 1)
    assert pool.num_free == 6 and len(pool.free_list()) == 2
    x, y = pool.alloc(), pool.alloc()                     # free list first: blocks 4 then 5
    assert (x, y) == (4, 5)
    # then the oldest unreferenced leaf: block 3 (its parent 2 is older but not a leaf)
    assert pool.alloc() == 3
    assert pool.alloc() == 2                              # 2 is now a leaf, stamp 1
    assert pool.alloc() == 1 and pool.alloc() == 0
    with pytest.raises(PoolError) as e:
        pool.alloc()
    assert e.value.status == ERR_NO_FREE_BLOCK


def test_write_into_cached_block_copies_it():
    pool = PrefixCachedPool(8, BS)
    t, lt = write_seq(pool, list(range(8)))
    pool.insert(list(range(8)), t, lt)
    old = t[1]
    lt2, plan = pool.plan_write(t, 16, lt, 6, 1)          # rewrite position 6 (block 1)
    assert plan.copies == [(old, t[1])] and t[1] != old
    assert pool.refcount[old] == 0 and pool.cached(old)   # the cached content is kept, unreferenced


def test_invalid_insert_changes_nothing():
    pool = PrefixCachedPool(8, BS)
    t, lt = write_seq(pool, list(range(8)))
    pool.insert(list(range(8)), t, lt)
    u, lu = write_seq(pool, [9] * 8)
    before = (pool.dump(), list(pool.refcount), pool.free_list())
    with pytest.raises(PoolError) as e:                   # t[0] is already cached under tokens 0..3
        pool.insert([9] * 4 + [8] * 4, [u[0], t[0]], 2)
    assert e.value.status == ERR_INVALID_ARG
    assert (pool.dump(), list(pool.refcount), pool.free_list()) == before


def check_invariants(pool, tables):
    nb = pool.num_blocks
    held = [0] * nb
    for tab, live in tables.values():
        for j in range(live):
            held[tab[j]] += 1
    assert pool.refcount == held
    free = pool.free_list()
    cached = {b for b, _, _ in pool.dump()}
    unref = {b for b, _, t in pool.dump() if t >= 0}
    assert len(free) == len(set(free)) and not (set(free) & cached)
    assert unref == {b for b in cached if pool.refcount[b] == 0}
    assert set(free) == {b for b in range(nb) if pool.refcount[b] == 0} - cached
    for b, par, _ in pool.dump():
        assert par == -1 or par in cached       # every cached block is reachable from the root
    # reclaimable: unreferenced blocks with no referenced descendant, by brute force
    desc = {b: set() for b in cached}
    for b in cached:
        x = pool.parent[b]
        while x is not None:
            desc[x].add(b)
            x = pool.parent[x]
    want = sum(1 for b in unref if all(pool.refcount[d] == 0 for d in desc[b]))
    assert pool.reclaimable() == want
    # draining the cache hands out exactly that many blocks
    probe = copy.deepcopy(pool)
    assert len(probe.evict(10 ** 6)) == want


@pytest.mark.parametrize("seed", range(4))
def test_random_request_stream_invariants_and_longest_match(seed):
    rng = np.random.default_rng(seed)
    pool = PrefixCachedPool(40, BS, initial_free_order=rng.permutation(40))
    prompts = [list(rng.integers(0, 3, size=int(rng.integers(4, 20)))) for _ in range(6)]
    tables = {}
    for step in range(300):
        op = rng.integers(0, 4)
        if op == 0 or not tables:                  # a new request: match, then write the rest
            sid = step
            toks = prompts[rng.integers(len(prompts))] + list(rng.integers(0, 3, size=int(rng.integers(0, 9))))
            tab = [-1] * 16
            m = pool.match(toks, 16)
            # brute force: every cached block's full token prefix, rebuilt from its
            # parent chain; the match is the longest of them that toks starts with
            prefixes = cached_prefixes(pool)
            best = max([len(pfx) // BS for pfx in prefixes if tuple(toks[:len(pfx)]) == pfx] + [0])
            assert len(m) == min(best, 16)
            tab[:len(m)] = m
            try:
                live, _ = pool.plan_write(tab, 16, len(m), len(m) * BS, len(toks) - len(m) * BS)
            except PoolError as e:
                assert e.status == ERR_NO_FREE_BLOCK
                for b in m:
                    pool.free(b)
                check_invariants(pool, {k: (v[0], v[1]) for k, v in tables.items()})
                continue
            tables[sid] = (tab, live, toks)
        elif op == 1:                              # a request caches its prompt blocks
            sid = list(tables)[rng.integers(len(tables))]
            tab, live, toks = tables[sid]
            try:
                pool.insert(toks, tab, live)
            except PoolError as e:
                assert e.status == ERR_INVALID_ARG
        elif op == 2:                              # a request finishes
            sid = list(tables)[rng.integers(len(tables))]
            tab, live, _ = tables.pop(sid)
            for j in range(live):
                pool.free(tab[j])
        else:                                      # memory pressure: evict some
            pool.evict(int(rng.integers(1, 4)))
        check_invariants(pool, {k: (v[0], v[1]) for k, v in tables.items()})


def cached_prefixes(pool):
    """Token prefix of every cached block: the keys along its parent chain."""
    parent = {b: par for b, par, _ in pool.dump()}
    out = set()
    for b in parent:
        chain, x = [], b
        while x != -1:
            chain.append(pool.key[x])
            x = parent[x]
        out.add(tuple(t for k in reversed(chain) for t in k))
    return out
