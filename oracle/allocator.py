"""Refcounted physical block pool with copy-on-write (pure-Python model).

What the pages fix:
  * The KV cache is cut into fixed-size physical blocks that may sit anywhere
    in device memory; a per-sequence block table maps logical block j (tokens
    j*bs .. j*bs+bs-1) to a physical block id ("AI & MLOps Blog #54", section
    2.2, logical->physical diagram; Part 8, "PagedAttention: Ảo Hóa Phân
    Trang ..." and the block-table diagram in "Phân Tích Cơ Cấu Bộ Nhớ").
  * A sequence takes one new block from the free pool each time it grows past
    a multiple of the block size (Blog #54, interview question 2).
  * Sequences that share a prompt point at the same physical blocks and the
    block's reference count equals the number of sharers (question 2: four
    parallel samples give a count of 4; Part 8, "RadixAttention": a reuse
    increments ref_count).
  * On divergence only the part being written gets a new private block
    (copy-on-write, question 2); blocks whose count reaches 0 are free again
    (Part 8, "RadixAttention").

What the pages leave open, and the reading taken here:
  * Which free block is handed out: the free list is a LIFO stack. Its initial
    order is given (a seeded permutation in the workloads, ascending by
    default), allocation pops the head, and a block whose count falls to 0 is
    pushed back on the head.
  * A write that touches a shared block copies it (all KV heads, K and V)
    into a fresh block, drops one reference from the old block and patches
    the table entry; blocks are processed in ascending logical order.
  * Errors leave the pool unchanged: a write first checks that the table has
    room and that the pool can supply every block it needs.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_NO_FREE_BLOCK = 3
ERR_BAD_BLOCK = 4


class PoolError(Exception):
    def __init__(self, status: int, msg: str = ""):
        super().__init__(f"status {status}: {msg}")
        self.status = status


@dataclass
class WritePlan:
    copies: List[Tuple[int, int]]     # (src block, dst block), in issue order
    slots: List[int]                  # physical slot (block*bs + offset) per token


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise PoolError(ERR_INVALID_ARG, "pool shape")
        order = list(range(num_blocks)) if initial_free_order is None else [int(x) for x in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError(ERR_INVALID_ARG, "initial free order is not a permutation")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.refcount = [0] * num_blocks
        # stack: the last element is the head of the free list
        self._stack = list(reversed(order))

    # -- queries -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._stack)

    def free_list(self) -> List[int]:
        """Free blocks from head (next to be handed out) to tail."""
        return list(reversed(self._stack))

    def _check(self, blk: int) -> None:
        if not (0 <= blk < self.num_blocks):
            raise PoolError(ERR_INVALID_ARG, f"block {blk} out of range")

    # -- single-block operations ------------------------------------------
    def alloc(self) -> int:
        if not self._stack:
            raise PoolError(ERR_NO_FREE_BLOCK, "pool exhausted")
        blk = self._stack.pop()
        self.refcount[blk] = 1
        return blk

    def fork(self, blk: int) -> None:
        self._check(blk)
        if self.refcount[blk] == 0:
            raise PoolError(ERR_BAD_BLOCK, f"fork of free block {blk}")
        self.refcount[blk] += 1

    def free(self, blk: int) -> None:
        self._check(blk)
        if self.refcount[blk] == 0:
            raise PoolError(ERR_BAD_BLOCK, f"free of free block {blk}")
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self._stack.append(blk)

    def _must_copy(self, blk: int) -> bool:
        """A write into blk copies it first: it has other readers."""
        return self.refcount[blk] > 1

    # -- appending / overwriting tokens of one sequence --------------------
    def plan_write(self, table: List[int], capacity: int, num_blocks: int,
                   start_pos: int, n_tokens: int) -> Tuple[int, WritePlan]:
        """Make room for tokens [start_pos, start_pos + n_tokens) of one sequence.

        ``table`` holds the sequence's physical ids (its first ``num_blocks``
        entries are live) and is patched in place. Returns the new live-block
        count and the plan: block copies to issue and each token's slot.
        """
        bs = self.block_size
        if start_pos < 0 or n_tokens < 0 or num_blocks < 0 or num_blocks > capacity:
            raise PoolError(ERR_INVALID_ARG, "negative position/count or bad table size")
        if n_tokens == 0:
            return num_blocks, WritePlan([], [])
        if start_pos > num_blocks * bs:
            raise PoolError(ERR_INVALID_ARG, "write would leave a hole in the table")
        end = start_pos + n_tokens
        last_block = (end - 1) // bs
        if last_block >= capacity:
            raise PoolError(ERR_INVALID_ARG, "block table too small")
        first_block = start_pos // bs
        for j in range(first_block, min(num_blocks, last_block + 1)):
            self._check(table[j])
            if self.refcount[table[j]] == 0:
                raise PoolError(ERR_BAD_BLOCK, f"table entry {j} names free block {table[j]}")
        need = max(0, last_block + 1 - num_blocks)
        need += sum(1 for j in range(first_block, min(num_blocks, last_block + 1))
                    if self._must_copy(table[j]))
        if need > self.num_free:
            raise PoolError(ERR_NO_FREE_BLOCK, "pool cannot supply the write")

        copies: List[Tuple[int, int]] = []
        for j in range(first_block, last_block + 1):
            if j < num_blocks:
                old = table[j]
                if self._must_copy(old):
                    new = self.alloc()
                    copies.append((old, new))
                    self.free(old)
                    table[j] = new
            else:
                table[j] = self.alloc()
                num_blocks += 1
        slots = [table[p // bs] * bs + p % bs for p in range(start_pos, end)]
        return num_blocks, WritePlan(copies, slots)
