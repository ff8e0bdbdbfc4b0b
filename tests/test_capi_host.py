"""The C-ABI library on the host: exported symbols, the allocator and write
plan bit-exact against the Python model, error paths and launch planning.
No device work is done here."""
import os
import re

import numpy as np
import pytest

import paged_kv_cache_218_amd as pa
from paged_kv_cache_218_amd import _lib
from oracle.allocator import BlockPoolModel, PoolError
from oracle.build import build_pool
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pagedattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "pa_attention" in names and "pa_write_kv" in names and len(names) >= 15
    for n in names:
        assert hasattr(_lib.lib, n), n
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == names


def test_status_strings():
    for s in range(8):
        assert pa.pa_status_string(s) != "unknown status"
    assert pa.pa_status_string(_lib.PA_ERR_NO_MEMORY) == "out of host memory"
    assert pa.pa_status_string(99) == "unknown status"


def test_pool_buffer_bytes():
    assert pa.pa_pool_buffer_bytes(16384, 32, 8, 128, pa.PA_DTYPE_BF16) == 2**30
    assert pa.pa_pool_buffer_bytes(32, 16, 2, 64, pa.PA_DTYPE_F32) == 32 * 16 * 2 * 64 * 4
    # FP8: one byte per element plus one fp32 scale per (block, head, slot)
    assert pa.pa_pool_buffer_bytes(16384, 32, 8, 128, pa.PA_DTYPE_FP8_E4M3) == 2**29 + 16384 * 8 * 32 * 4
    assert pa.pa_pool_buffer_bytes(16, 8, 2, 64, pa.PA_DTYPE_BF16) == -1
    assert pa.pa_pool_buffer_bytes(16, 16, 2, 64, 9) == -1


def test_kv_bytes_per_token_matches_closed_form():
    assert pa.pa_kv_bytes_per_token(80, 8, 128, 2) == 327680
    assert pa.pa_kv_bytes_per_token(1, 8, 128, 2) == 4096
    assert pa.pa_kv_bytes_per_token(32, 8, 128, 4) == 262144
    assert pa.pa_kv_bytes_per_token(0, 8, 128, 2) == -1


def state(pool, nb):
    return [pa.pa_block_refcount(pool, b) for b in range(nb)], list(pa.pa_pool_free_list(pool))


def model_state(m):
    return list(m.refcount), m.free_list()


def test_random_alloc_fork_free_bit_exact():
    rng = np.random.default_rng(11)
    nb = 40
    order = rng.permutation(nb).astype(np.int32)
    pool = pa.pa_pool_create(nb, 16, 2, 64, pa.PA_DTYPE_BF16, order)
    m = BlockPoolModel(nb, 16, order)
    live = []
    for step in range(3000):
        op = rng.integers(0, 3)
        if op == 0:
            try:
                want = m.alloc()
            except PoolError as e:
                with pytest.raises(pa.PAError) as ex:
                    pa.pa_block_alloc(pool)
                assert ex.value.status == e.status
                continue
            assert pa.pa_block_alloc(pool) == want
            live.append(want)
        elif op == 1 and live:
            b = int(rng.choice(live))
            m.fork(b)
            pa.pa_block_fork(pool, b)
            live.append(b)
        elif op == 2 and live:
            b = live.pop(int(rng.integers(len(live))))
            m.free(b)
            pa.pa_block_free(pool, b)
        if step % 97 == 0:
            assert state(pool, nb) == model_state(m)
    assert state(pool, nb) == model_state(m)


def test_error_statuses_match_model_and_leave_state():
    pool = pa.pa_pool_create(3, 16, 2, 64, pa.PA_DTYPE_F32)
    b = pa.pa_block_alloc(pool)
    pa.pa_block_free(pool, b)
    snap = state(pool, 3)
    for fn, arg, status in [(pa.pa_block_free, b, _lib.PA_ERR_BAD_BLOCK),
                            (pa.pa_block_fork, b, _lib.PA_ERR_BAD_BLOCK),
                            (pa.pa_block_free, 7, _lib.PA_ERR_INVALID_ARG),
                            (pa.pa_block_fork, -1, _lib.PA_ERR_INVALID_ARG)]:
        with pytest.raises(pa.PAError) as e:
            fn(pool, arg)
        assert e.value.status == status
    assert state(pool, 3) == snap
    for _ in range(3):
        pa.pa_block_alloc(pool)
    with pytest.raises(pa.PAError) as e:
        pa.pa_block_alloc(pool)
    assert e.value.status == _lib.PA_ERR_NO_FREE_BLOCK


def test_pool_create_validation():
    for args, status in [((0, 16, 2, 64, 0), _lib.PA_ERR_INVALID_ARG),
                         ((8, 8, 2, 64, 0), _lib.PA_ERR_UNSUPPORTED),
                         ((8, 16, 2, 96, 0), _lib.PA_ERR_UNSUPPORTED),
                         ((8, 16, 2, 64, 5), _lib.PA_ERR_UNSUPPORTED)]:
        with pytest.raises(pa.PAError) as e:
            pa.pa_pool_create(*args)
        assert e.value.status == status
    with pytest.raises(pa.PAError) as e:
        pa.pa_pool_create(4, 16, 2, 64, 0, [0, 1, 1, 2])
    assert e.value.status == _lib.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_write_plans_bit_exact(seed):
    """Sequences grow, fork prefixes, overwrite, and free, through both sides."""
    rng = np.random.default_rng(100 + seed)
    nb, bs, cap, nseq = 64, 16, 12, 6
    order = rng.permutation(nb).astype(np.int32)
    pool = pa.pa_pool_create(nb, bs, 2, 64, pa.PA_DTYPE_BF16, order)
    m = BlockPoolModel(nb, bs, order)
    tab_c = np.full((nseq, cap), -1, dtype=np.int32)
    tab_m = [[-1] * cap for _ in range(nseq)]
    live = [0] * nseq
    length = [0] * nseq
    for step in range(400):
        s = int(rng.integers(nseq))
        op = rng.integers(0, 10)
        if op < 6:       # append or overwrite a few tokens
            start = int(rng.integers(max(0, length[s] - 20), length[s] + 1))
            n = int(rng.integers(1, 40))
            try:
                lm, plan = m.plan_write(tab_m[s], cap, live[s], start, n)
            except PoolError as e:
                row = tab_c[s].copy()
                with pytest.raises(pa.PAError) as ex:
                    pa.pa_write_plan(pool, tab_c[s], live[s], start, n)
                assert ex.value.status == e.status
                assert np.array_equal(tab_c[s], row)
                continue
            lc, copies, slots = pa.pa_write_plan(pool, tab_c[s], live[s], start, n)
            assert lc == lm and copies == plan.copies and list(slots) == plan.slots
            live[s] = lm
            length[s] = max(length[s], start + n)
        elif op < 8:     # another sequence adopts this one's blocks (prefix sharing)
            d = int(rng.integers(nseq))
            if d == s or live[s] == 0:
                continue
            for j in range(live[d]):
                m.free(tab_m[d][j])
                pa.pa_block_free(pool, int(tab_c[d, j]))
            for j in range(live[s]):
                m.fork(tab_m[s][j])
                pa.pa_block_fork(pool, int(tab_c[s, j]))
            tab_m[d] = list(tab_m[s])
            tab_c[d] = tab_c[s]
            live[d], length[d] = live[s], length[s]
        else:            # the sequence finishes
            for j in range(live[s]):
                m.free(tab_m[s][j])
                pa.pa_block_free(pool, int(tab_c[s, j]))
            tab_m[s] = [-1] * cap
            tab_c[s] = -1
            live[s] = length[s] = 0
        assert [list(r[:l]) for r, l in zip(tab_c, live)] == [r[:l] for r, l in zip(tab_m, live)]
    assert state(pool, nb) == model_state(m)


@pytest.mark.parametrize("name,kw", [
    ("prefix_verify", dict(batch=5, prefix_len=40, len_lo=20, len_hi=70)),
    ("prefix_verify", dict(batch=5, prefix_len=32, len_lo=20, len_hi=70)),
    ("llama3_8b_decode", dict(batch=6, len_lo=30, len_hi=300)),
])
def test_workload_tables_bit_exact(name, kw):
    """The fixed build order of a workload gives the same tables and refcounts."""
    w = workloads.generate(workloads.config(name, **kw))
    cfg = w.cfg
    _, m, tables, live = build_pool(w)
    pool = pa.pa_pool_create(w.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim,
                             pa.PA_DTYPE_BF16, w.free_order)
    tab = np.full((cfg.batch, w.max_blocks), -1, dtype=np.int32)
    lv = [0] * cfg.batch
    if cfg.prefix_len:
        lv[0], _, _ = pa.pa_write_plan(pool, tab[0], 0, 0, cfg.prefix_len)
        for b in range(1, cfg.batch):
            for j in range(lv[0]):
                pa.pa_block_fork(pool, int(tab[0, j]))
            tab[b, :lv[0]] = tab[0, :lv[0]]
            lv[b] = lv[0]
    for b in range(cfg.batch):
        lv[b], _, _ = pa.pa_write_plan(pool, tab[b], lv[b], cfg.prefix_len, int(w.lens[b]) - cfg.prefix_len)
    assert np.array_equal(tab, tables) and lv == live
    assert state(pool, w.num_blocks) == model_state(m)


def test_attention_plan_validation():
    ok = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
              max_blocks_per_seq=8, num_blocks=32, dtype=pa.PA_DTYPE_BF16, max_context=128)
    pl = pa.pa_attention_plan(pa.make_desc(**ok), 1)
    assert pl.path == pa.PA_PATH_MFMA and pl.schedule == _lib.PA_SCHED_BALANCED
    assert pl.waves_per_group == 4 and pl.tiles_per_wave == 1
    # contexts of 2048 tokens or more: one workgroup of 8 waves per compute unit (with one
    # row tile 12 would fit, 8 measure faster), except two FP8 tiles (two workgroups of 4);
    # 12 waves stay available on request
    long_ctx = {**ok, "max_context": 2048, "max_blocks_per_seq": 512}
    pl_long = pa.pa_attention_plan(pa.make_desc(**long_ctx), 1)
    assert pl_long.waves_per_group == 8 and pl_long.tiles_per_wave == 1
    assert pa.pa_attention_plan(pa.make_desc(**{**long_ctx, "waves_per_group": 12}), 1).waves_per_group == 12
    pl_long = pa.pa_attention_plan(pa.make_desc(**{**long_ctx, "num_q_heads": 40}), 1)
    assert pl_long.waves_per_group == 8 and pl_long.tiles_per_wave == 2
    pl_long = pa.pa_attention_plan(pa.make_desc(**{**long_ctx, "num_q_heads": 40,
                                                  "kv_format": pa.PA_KV_FP8_E4M3}), 1)
    assert pl_long.waves_per_group == 4 and pl_long.tiles_per_wave == 2
    # a segment's start counts for 8 steps over bf16 pools, 16 over FP8 (half the bytes a step)
    assert pl.segment_cost == 8 and pl_long.segment_cost == 16
    assert pa.pa_attention_plan(pa.make_desc(**{**long_ctx, "max_context": 2047}), 1).waves_per_group == 4
    assert pa.pa_attention_plan(pa.make_desc(**{**long_ctx, "num_q_heads": 40, "waves_per_group": 8}),
                                1).waves_per_group == 8
    # 8 waves' park area for 32 rows plus 8192 sequences' step sums exceed the LDS
    big = {**ok, "num_seqs": 8192, "num_q_heads": 64}
    assert pa.pa_attention_plan(pa.make_desc(**big), 1).waves_per_group == 4
    with pytest.raises(pa.PAError) as e:
        pa.pa_attention_plan(pa.make_desc(**{**big, "waves_per_group": 8}), 1)
    assert e.value.status == _lib.PA_ERR_UNSUPPORTED
    assert pl.workspace_bytes == pa.pa_attention_workspace_size(pa.make_desc(**ok), 1) > 0
    pl = pa.pa_attention_plan(pa.make_desc(**{**ok, "partition_tokens": 64}), 1)
    assert pl.schedule == _lib.PA_SCHED_PARTITIONS and pl.num_partitions == 2 and pl.segment_cost == 0
    pl = pa.pa_attention_plan(pa.make_desc(**{**ok, "path": pa.PA_PATH_VALU}), 1)
    assert pl.schedule == _lib.PA_SCHED_PARTITIONS
    # partitions that fill the device's 3072 wave slots on their own: one wavefront each,
    # and with more partitions than slots (8,192 here) runs of 3 consecutive partitions per
    # wavefront: ceil(256 / 3) = 86 runs per (sequence, KV head), 4 wavefronts per workgroup
    many = {**ok, "num_seqs": 4, "num_kv_heads": 8, "num_q_heads": 64, "block_size": 32,
            "max_context": 131072, "max_blocks_per_seq": 4096, "num_blocks": 16384, "partition_tokens": 512}
    pl = pa.pa_attention_plan(pa.make_desc(**many), 1)
    assert pl.schedule == _lib.PA_SCHED_PARTITIONS_WAVE and pl.num_partitions == 256
    assert pl.grid == 32 * 86 // 4 and pl.merge_grid == 4 * 64 and pl.partitions_per_wave == 3
    rows_parts = 4 * 64 * 256
    # the balanced schedule's counter area (4 x 8 pairs, one 256-byte unit) comes first in every layout
    assert pl.workspace_bytes == 256 + -(-rows_parts * 8 // 256) * 256 + rows_parts * 128 * 4
    # partitions that exactly fill the slots: one wavefront each
    exact = {**many, "num_seqs": 3, "max_context": 65536, "max_blocks_per_seq": 2048}
    pl = pa.pa_attention_plan(pa.make_desc(**exact), 1)  # 24 pairs x 128 partitions = 3072 slots
    assert pl.schedule == _lib.PA_SCHED_PARTITIONS_WAVE and pl.grid == 24 * 128 // 4 and pl.partitions_per_wave == 1
    assert pa.pa_attention_plan(pa.make_desc(**{**many, "max_context": 3072 * 512 // 32 - 512}),
                                1).schedule == _lib.PA_SCHED_PARTITIONS
    assert pa.pa_attention_plan(pa.make_desc(**{**many, "path": pa.PA_PATH_VALU}),
                                1).schedule == _lib.PA_SCHED_PARTITIONS
    bad = [
        (dict(num_q_heads=7), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(head_dim=96), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(block_size=8), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(max_context=129), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(), 0, _lib.PA_ERR_INVALID_ARG),
        (dict(), 129, _lib.PA_ERR_INVALID_ARG),
        (dict(partition_tokens=100), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(dtype=7), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(num_q_heads=80, num_kv_heads=2), 1, _lib.PA_ERR_UNSUPPORTED),   # 40 rows
        (dict(dtype=pa.PA_DTYPE_F32, path=pa.PA_PATH_MFMA), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(waves_per_group=3), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(waves_per_group=16), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(waves_per_group=8, partition_tokens=64), 1, _lib.PA_ERR_UNSUPPORTED),   # partition kernels: <= 4
        (dict(waves_per_group=12, num_q_heads=40, num_kv_heads=2), 1, _lib.PA_ERR_UNSUPPORTED),  # two tiles: <= 8
        (dict(kv_format=2), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(kv_format=pa.PA_KV_FP8_E4M3, path=pa.PA_PATH_VALU), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(kv_format=pa.PA_KV_FP8_E4M3, dtype=pa.PA_DTYPE_F32), 1, _lib.PA_ERR_UNSUPPORTED),
        (dict(num_seqs=0), 1, _lib.PA_ERR_INVALID_ARG),            # empty batch
        (dict(num_kv_heads=0), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(num_blocks=0), 1, _lib.PA_ERR_INVALID_ARG),          # empty pool
        (dict(max_blocks_per_seq=0), 1, _lib.PA_ERR_INVALID_ARG),
        (dict(max_context=0), 1, _lib.PA_ERR_INVALID_ARG),
    ]
    for over, q_len, status in bad:
        with pytest.raises(pa.PAError) as e:
            pa.pa_attention_plan(pa.make_desc(**{**ok, **over}), q_len)
        assert e.value.status == status, (over, q_len)
    # the workloads' own partitioning
    d = pa.make_desc(4, 64, 8, 128, 32, 4096, 16384, pa.PA_DTYPE_BF16, 131072, partition_tokens=512)
    pl = pa.pa_attention_plan(d, 1)
    assert (pl.num_partitions, pl.merge_grid) == (256, 4 * 64)
    assert pl.workspace_bytes == 256 + 4 * 64 * 256 * (128 + 2) * 4
    assert pa.pa_attention_workspace_size(d, 1) == pl.workspace_bytes


def test_tree_masks_bit_exact_vs_oracle():
    from oracle import tree as otree
    rng = np.random.default_rng(11)
    for n in (1, 2, 5, 8, 17, 32):
        for _ in range(20):
            parents = [int(rng.integers(-1, j)) for j in range(n)]
            got = pa.pa_tree_masks(np.array(parents, dtype=np.int32))
            assert got.tolist() == otree.ancestor_masks(parents)


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 2, 0], [-2], list(range(-1, 32))])
def test_tree_masks_errors(bad):
    with pytest.raises(pa.PAError) as ex:
        pa.pa_tree_masks(np.array(bad, dtype=np.int32))
    assert ex.value.status == _lib.PA_ERR_INVALID_ARG


def test_attention_tree_rejects_bad_masks_before_launch():
    """Argument checks of the tree entry point return before any device work
    (the pointers below are never dereferenced)."""
    import ctypes as C
    desc = pa.make_desc(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        max_blocks_per_seq=8, num_blocks=32, dtype=pa.PA_DTYPE_BF16, max_context=128)
    fake = 256

    def call(q_len, mask, stride):
        return _lib.lib.pa_attention_tree(C.byref(desc), fake, fake, fake, fake, fake, q_len, mask, stride,
                                          1.0, fake, None, 0, None)
    assert call(4, None, 4) == _lib.PA_ERR_INVALID_ARG          # no masks
    assert call(33, fake, 33) == _lib.PA_ERR_INVALID_ARG        # more nodes than mask bits
    assert call(4, fake, 3) == _lib.PA_ERR_INVALID_ARG          # rows of one sequence overlap the next
    assert call(4, fake, -1) == _lib.PA_ERR_INVALID_ARG
    assert call(0, fake, 0) == _lib.PA_ERR_INVALID_ARG


def test_attention_rejects_small_or_misaligned_workspace_before_launch():
    """The split-KV partials need a workspace of the reported size, 16-byte
    aligned; anything else is refused before any device work (the pointers
    below are never dereferenced)."""
    import ctypes as C
    desc = pa.make_desc(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        max_blocks_per_seq=8, num_blocks=32, dtype=pa.PA_DTYPE_BF16, max_context=128,
                        partition_tokens=64)
    size = pa.pa_attention_workspace_size(desc, 1)
    assert size > 0
    fake = 256

    def call(ws, nbytes):
        return _lib.lib.pa_attention(C.byref(desc), fake, fake, fake, fake, fake, 1, 1.0, fake, ws, nbytes, None)
    assert call(None, size) == _lib.PA_ERR_INVALID_ARG          # no workspace
    assert call(4096, size - 1) == _lib.PA_ERR_INVALID_ARG      # too small
    assert call(4096 + 8, size) == _lib.PA_ERR_INVALID_ARG      # 8-byte aligned only
    assert _lib.lib.pa_attention(C.byref(desc), fake, fake, fake, fake, fake, 1, float("nan"), fake, 4096,
                                 size, None) == _lib.PA_ERR_INVALID_ARG


def test_noalloc_refuses_more_than_its_scratch_before_device_work():
    """pa_attention_noalloc holds PA_NOALLOC_SCRATCH_BYTES of scratch; a call
    whose split-KV state needs more is refused with PA_ERR_TOO_LARGE, and bad
    arguments as pa_attention refuses them, all before any device work (the
    pointers below are never dereferenced)."""
    import ctypes as C
    fake = 256
    # 64 x 64 rows, 2,048 partitions of 64 tokens: 4,096 x 2,048 x 130 x 4 B of partials
    big = pa.make_desc(64, 64, 8, 128, 32, 4096, 16384, pa.PA_DTYPE_BF16, 131072, partition_tokens=64)
    assert pa.pa_attention_workspace_size(big, 1) > _lib.PA_NOALLOC_SCRATCH_BYTES
    call = lambda d, scale=1.0: _lib.lib.pa_attention_noalloc(C.byref(d), fake, fake, fake, fake, fake, 1, scale,
                                                              fake, None)
    assert call(big) == _lib.PA_ERR_TOO_LARGE
    assert pa.pa_status_string(_lib.PA_ERR_TOO_LARGE).startswith("needs more scratch")
    assert call(big, float("nan")) == _lib.PA_ERR_INVALID_ARG
    bad = pa.make_desc(64, 60, 8, 128, 32, 4096, 16384, pa.PA_DTYPE_BF16, 131072)   # 60 % 8 != 0
    assert call(bad) == _lib.PA_ERR_INVALID_ARG
    assert _lib.lib.pa_attention_noalloc(C.byref(big), None, fake, fake, fake, fake, 1, 1.0, fake,
                                         None) == _lib.PA_ERR_INVALID_ARG


def test_one_hip_runtime_per_process():
    """Importing the package before torch must not load a second HIP runtime."""
    import subprocess
    import sys
    code = ("import paged_kv_cache_218_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_spec_accept_rejects_bad_arguments_before_launch():
    import ctypes as C
    fake = 256
    ws = pa.pa_spec_accept_workspace_size(4, 100)
    assert ws > 0 and pa.pa_spec_accept_workspace_size(0, 100) == 0
    call = lambda *a: _lib.lib.pa_spec_accept(*a)
    for args in [(fake, fake, fake, fake, fake, 0, 5, 100, fake, fake, fake, ws, None),
                 (fake, fake, fake, fake, fake, 4, -1, 100, fake, fake, fake, ws, None),
                 (fake, fake, fake, fake, fake, 4, 5, 0, fake, fake, fake, ws, None),
                 (None, fake, fake, fake, fake, 4, 5, 100, fake, fake, fake, ws, None),
                 (fake, None, fake, fake, fake, 4, 5, 100, fake, fake, fake, ws, None),
                 (fake, fake, fake, fake, None, 4, 5, 100, fake, fake, fake, ws, None),
                 (fake, fake, fake, fake, fake, 4, 5, 100, None, fake, fake, ws, None),
                 (fake, fake, fake, fake, fake, 4, 5, 100, fake, fake, None, ws, None),
                 (fake, fake, fake, fake, fake, 4, 5, 100, fake, fake, fake, ws - 1, None)]:
        assert call(*args) == _lib.PA_ERR_INVALID_ARG, args


def test_read_probe_rejects_bad_arguments_before_launch():
    fake = 256
    call = lambda *a: _lib.lib.pa_read_probe(*a)
    for args in [(None, 4, 8192, fake, 1, 8, fake, None), (fake, 4, 8192, None, 1, 8, fake, None),
                 (fake, 4, 8192, fake, 1, 8, None, None), (fake, 0, 8192, fake, 1, 8, fake, None),
                 (fake, 4, 8192, fake, 1, 0, fake, None), (fake, 4, 8192, fake, 3, 8, fake, None),
                 (fake, 4, 2048, fake, 1, 8, fake, None), (fake, 4, 8193, fake, 1, 8, fake, None)]:
        assert call(*args) == _lib.PA_ERR_INVALID_ARG, args


def test_handles_alive_at_interpreter_exit_release_quietly():
    """A pool and a prefix cache still referenced by module globals when the
    interpreter exits are destroyed without errors from their finalizers."""
    import subprocess
    import sys
    code = ("import paged_kv_cache_218_amd as pa\n"
            "pool = pa.pa_pool_create(8, 16, 2, 64, pa.PA_DTYPE_BF16)\n"
            "cache = pa.pa_prefix_cache_create(pool)\n"
            "blk = pa.pa_block_alloc(pool)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "Exception ignored" not in r.stderr and "Error" not in r.stderr, r.stderr
