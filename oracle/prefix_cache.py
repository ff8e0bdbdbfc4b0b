"""Radix-tree prefix cache over the block pool (pure-Python model). TEST
INFRASTRUCTURE ONLY.

Part 8, "RadixAttention": the KV blocks of earlier requests are kept in a
prefix tree; a new request whose tokens match a cached prefix reuses those
physical blocks by incrementing their reference counts and skips their
prefill; under memory pressure an LRU policy frees blocks whose count is 0.
"Mở rộng Quy mô và Triển khai", "Cache Tiền tố": the longest cached prefix is
found and generation starts from there.

Readings taken (the pages give the policy, not the mechanics):
  * granularity: one tree node per full block, keyed by that block's
    block_size token ids; children of a node continue its prefix. A
    partial block is never cached, since it is still being written;
  * a cached block whose count falls to 0 is not returned to the free list:
    it stays in the tree, unreferenced and reclaimable, stamped with the time
    (a counter bumped by every such event) at which it became unreferenced;
  * allocation takes the free list first; when it is empty, the unreferenced
    leaf with the oldest stamp is evicted from the tree and handed out. Only
    leaves are evicted, so every cached block stays reachable through its
    parent; an unreferenced parent becomes a leaf when its last child goes.
    A block is reclaimable when it and its whole subtree are unreferenced
    (a request may hold a cached block without its parent: insertion follows
    an existing node with the same tokens, and a write copies a cached block
    out of a request's table);
  * matching forks each matched block (0 -> 1 revives an unreferenced one)
    and writes it into the request's table; at most the table's capacity;
  * insertion walks the request's full blocks: an existing child with the
    same tokens is followed, otherwise the request's own block becomes that
    child. A block already in the tree under another prefix, or a free block,
    makes the insertion invalid (nothing changes);
  * a write into a cached block copies it first even when its count is 1, so
    cached contents never change under a reader;
  * explicit eviction returns up to n evicted blocks to the free list's head,
    in eviction order.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from .allocator import (ERR_BAD_BLOCK, ERR_INVALID_ARG, ERR_NO_FREE_BLOCK, BlockPoolModel,
                        PoolError)


class PrefixCachedPool(BlockPoolModel):
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        super().__init__(num_blocks, block_size, initial_free_order)
        self.clock = 0
        self.children: Dict[Optional[int], Dict[Tuple[int, ...], int]] = {None: {}}
        self.parent: Dict[int, Optional[int]] = {}
        self.key: Dict[int, Tuple[int, ...]] = {}
        self.unref_time: Dict[int, int] = {}       # unreferenced cached blocks

    # -- state ---------------------------------------------------------------
    def cached(self, blk: int) -> bool:
        return blk in self.key

    @property
    def num_free(self) -> int:
        """Blocks an allocation can obtain: the free list plus every cached
        block whose whole subtree is unreferenced (each becomes an evictable
        leaf in turn; a block with a referenced descendant never does)."""
        return len(self._stack) + self.reclaimable()

    def reclaimable(self) -> int:
        count = 0
        live_below: Dict[int, bool] = {}
        order, stack = [], [None]
        while stack:                                   # preorder, then children before parents
            node = stack.pop()
            order.append(node)
            stack.extend(self.children[node].values())
        for node in reversed(order):
            live = any(live_below[c] for c in self.children[node].values())
            if node is not None:
                if self.refcount[node] > 0:
                    live = True
                elif not live:
                    count += 1
                live_below[node] = live
        return count

    def _must_copy(self, blk: int) -> bool:
        return self.refcount[blk] > 1 or self.cached(blk)

    def _evict_one(self) -> int:
        leaves = [b for b in self.unref_time if not self.children[b]]
        victim = min(leaves, key=lambda b: (self.unref_time[b], b))
        del self.children[self.parent[victim]][self.key[victim]]
        del self.children[victim], self.parent[victim], self.key[victim], self.unref_time[victim]
        return victim

    # -- pool operations with the cache ---------------------------------------
    def alloc(self) -> int:
        if self._stack:
            return super().alloc()
        if not any(not self.children[b] for b in self.unref_time):
            raise PoolError(ERR_NO_FREE_BLOCK, "pool exhausted")
        blk = self._evict_one()
        self.refcount[blk] = 1
        return blk

    def free(self, blk: int) -> None:
        self._check(blk)
        if self.refcount[blk] == 0:
            raise PoolError(ERR_BAD_BLOCK, f"free of free block {blk}")
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            if self.cached(blk):
                self.clock += 1
                self.unref_time[blk] = self.clock
            else:
                self._stack.append(blk)

    # -- cache operations ----------------------------------------------------
    def match(self, tokens: Sequence[int], capacity: int) -> List[int]:
        """Longest cached prefix of whole blocks (at most capacity); forks them."""
        bs = self.block_size
        node: Optional[int] = None
        out: List[int] = []
        for i in range(min(len(tokens) // bs, capacity)):
            child = self.children[node].get(tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]))
            if child is None:
                break
            out.append(child)
            node = child
        for blk in out:
            if self.refcount[blk] == 0:
                del self.unref_time[blk]
            self.refcount[blk] += 1
        return out

    def insert(self, tokens: Sequence[int], table: Sequence[int], num_blocks: int) -> int:
        """Cache the request's full blocks; returns the number of new nodes."""
        bs = self.block_size
        n = min(num_blocks, len(tokens) // bs)
        node: Optional[int] = None
        plan: List[Tuple[Optional[int], Tuple[int, ...], int]] = []
        for i in range(n):
            chunk = tuple(int(t) for t in tokens[i * bs:(i + 1) * bs])
            child = self.children.get(node, {}).get(chunk)   # a planned node has no children yet
            if child is None:
                blk = int(table[i])
                self._check(blk)
                if self.refcount[blk] == 0:
                    raise PoolError(ERR_BAD_BLOCK, f"insert of free block {blk}")
                if self.cached(blk) or any(b == blk for _, _, b in plan):
                    raise PoolError(ERR_INVALID_ARG, f"block {blk} is cached under another prefix")
                plan.append((node, chunk, blk))
                node = blk
            else:
                node = child
        for par, chunk, blk in plan:
            self.children[par][chunk] = blk
            self.children[blk] = {}
            self.parent[blk] = par
            self.key[blk] = chunk
        return len(plan)

    def evict(self, max_blocks: int) -> List[int]:
        out = []
        while len(out) < max_blocks and any(not self.children[b] for b in self.unref_time):
            blk = self._evict_one()
            self._stack.append(blk)
            out.append(blk)
        return out

    def dump(self) -> List[Tuple[int, int, int]]:
        """(block, parent block or -1, unreferenced stamp or -1) per cached block, ascending."""
        return [(b, -1 if self.parent[b] is None else self.parent[b], self.unref_time.get(b, -1))
                for b in sorted(self.key)]
