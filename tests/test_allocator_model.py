"""The allocator model against the pages' narrative of paged block sharing."""
import pytest

from oracle.allocator import (ERR_BAD_BLOCK, ERR_INVALID_ARG, ERR_NO_FREE_BLOCK,
                              BlockPoolModel, PoolError)


def snapshot(m):
    return (list(m.refcount), m.free_list())


def test_growth_takes_one_block_per_block_size_tokens():
    # Blog #54 question 2: a sequence requests a new block each time it grows by bs tokens
    m = BlockPoolModel(8, 16)
    table, live = [-1] * 8, 0
    allocated_at = []
    for pos in range(70):
        before = m.num_free
        live, plan = m.plan_write(table, 8, live, pos, 1)
        if m.num_free != before:
            allocated_at.append(pos)
        assert plan.copies == []
    assert allocated_at == [0, 16, 32, 48, 64]
    assert live == 5 and table[:5] == [0, 1, 2, 3, 4]


def test_initial_free_order_and_lifo_reuse():
    m = BlockPoolModel(5, 4, initial_free_order=[3, 1, 4, 0, 2])
    got = [m.alloc() for _ in range(3)]
    assert got == [3, 1, 4]
    m.free(1)
    m.free(3)
    assert m.free_list() == [3, 1, 0, 2]
    assert m.alloc() == 3 and m.alloc() == 1


def test_four_samples_share_prompt_then_copy_only_the_diverging_block():
    # Blog #54 question 2: four answers to one prompt point at the prompt's blocks
    # (reference count 4); when they diverge only the part being written gets a
    # new block (copy-on-write).
    bs = 16
    m = BlockPoolModel(32, bs)
    t0, live0 = [-1] * 8, 0
    live0, _ = m.plan_write(t0, 8, live0, 0, 40)       # prompt: 40 tokens -> blocks 0,1,2 (2 is partial)
    assert t0[:3] == [0, 1, 2]
    tables = [t0] + [list(t0) for _ in range(3)]
    for t in tables[1:]:
        for j in range(3):
            m.fork(t[j])
    assert [m.refcount[b] for b in (0, 1, 2)] == [4, 4, 4]
    copies_per_seq = []
    for s, t in enumerate(tables):
        live, plan = m.plan_write(t, 8, 3, 40, 1)     # first generated token lands in block 2
        copies_per_seq.append(plan.copies)
        assert plan.slots == [t[2] * bs + 8]
    # the first three writers copy block 2; the last one is its sole owner by then
    assert [len(c) for c in copies_per_seq] == [1, 1, 1, 0]
    assert all(c[0][0] == 2 for c in copies_per_seq[:3])
    assert [t[2] for t in tables] == [3, 4, 5, 2]
    assert [m.refcount[b] for b in (0, 1, 2, 3, 4, 5)] == [4, 4, 1, 1, 1, 1]


def test_blocks_return_to_the_pool_at_refcount_zero():
    # Part 8 "RadixAttention": blocks whose ref_count is 0 can be reclaimed
    m = BlockPoolModel(6, 4)
    b = m.alloc()
    m.fork(b)
    m.fork(b)
    m.free(b)
    m.free(b)
    assert m.refcount[b] == 1 and b not in m.free_list()
    m.free(b)
    assert m.refcount[b] == 0 and m.free_list()[0] == b


def test_errors_leave_state_unchanged():
    m = BlockPoolModel(3, 4)
    t, live = [-1] * 4, 0
    live, _ = m.plan_write(t, 4, live, 0, 8)        # two blocks
    snap = snapshot(m)
    tsnap = list(t)
    with pytest.raises(PoolError) as e:
        m.plan_write(t, 4, live, 8, 8)              # needs 2 more blocks, 1 free
    assert e.value.status == ERR_NO_FREE_BLOCK
    assert snapshot(m) == snap and t == tsnap
    with pytest.raises(PoolError) as e:
        m.plan_write(t, 4, live, 8, 100)            # beyond the table's capacity
    assert e.value.status == ERR_INVALID_ARG
    with pytest.raises(PoolError) as e:
        m.plan_write(t, 4, live, 13, 1)             # would skip position 8..12
    assert e.value.status == ERR_INVALID_ARG
    free_blk = m.free_list()[0]
    with pytest.raises(PoolError) as e:
        m.fork(free_blk)
    assert e.value.status == ERR_BAD_BLOCK
    with pytest.raises(PoolError) as e:
        m.free(free_blk)
    assert e.value.status == ERR_BAD_BLOCK
    with pytest.raises(PoolError) as e:
        m.free(99)
    assert e.value.status == ERR_INVALID_ARG
    assert snapshot(m) == snap
    m.alloc()
    with pytest.raises(PoolError) as e:
        m.alloc()
    assert e.value.status == ERR_NO_FREE_BLOCK


def test_copy_on_write_only_for_shared_blocks_touched():
    m = BlockPoolModel(16, 4)
    t, live = [-1] * 8, 0
    live, _ = m.plan_write(t, 8, live, 0, 12)      # blocks 0,1,2 full
    other = list(t)
    for j in range(3):
        m.fork(other[j])
    # overwrite positions 5..9 (blocks 1 and 2) of the first sequence
    live, plan = m.plan_write(t, 8, live, 5, 5)
    assert plan.copies == [(1, 3), (2, 4)]
    assert t[:3] == [0, 3, 4] and other[:3] == [0, 1, 2]
    assert [m.refcount[b] for b in range(5)] == [2, 1, 1, 1, 1]
