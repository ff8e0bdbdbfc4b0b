"""HIP path vs the fp64 oracle through the C ABI (MI355X)."""
import numpy as np
import pytest

import workloads
from oracle.build import build_pool
from oracle.numerics import to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import (assert_close, assert_paths_agree, oracle_out, oracle_rows, out_bits,  # noqa: E402
                            out_to_f64, run_gpu)

VALU, MFMA = 1, 2

SMALL = {
    "tiny_f32": ("tiny_f32", dict()),
    "8b": ("llama3_8b_decode", dict(batch=5, len_lo=17, len_hi=700)),
    "70b": ("llama3_70b_decode", dict(batch=3, len_const=333)),
    "verify": ("prefix_verify", dict(batch=6, prefix_len=40, len_lo=20, len_hi=300)),
    "verify_aligned": ("prefix_verify", dict(batch=5, prefix_len=64, len_lo=5, len_hi=200)),
    "long": ("long_ctx_split", dict(batch=2, len_const=3000)),
    "70b_fp8": ("llama3_70b_decode_fp8", dict(batch=3, len_const=333)),
    "8b_fp8": ("llama3_8b_decode", dict(batch=5, len_lo=17, len_hi=700, kv_dtype="fp8")),
    "verify_fp8": ("prefix_verify", dict(batch=6, prefix_len=40, len_lo=20, len_hi=300, kv_dtype="fp8")),
    "long_fp8": ("long_ctx_split", dict(batch=2, len_const=3000, kv_dtype="fp8")),
    "d64_fp8": ("llama3_70b_decode_fp8", dict(batch=3, len_const=0, lens=(1, 64, 77), head_dim=64,
                                              num_q_heads=16, num_kv_heads=4)),
}
_cache = {}


def small(key):
    if key not in _cache:
        name, kw = SMALL[key]
        w = workloads.generate(workloads.config(name, **kw))
        _cache[key] = (w, oracle_out(w))
    return _cache[key]


CASES = [
    ("tiny_f32", VALU, 0), ("tiny_f32", VALU, 64),
    ("8b", MFMA, 0), ("8b", VALU, 0), ("8b", MFMA, 128), ("8b", VALU, 192),
    ("70b", MFMA, 0), ("70b", VALU, 0), ("70b", MFMA, 64),
    ("verify", MFMA, 0), ("verify", MFMA, 64), ("verify_aligned", MFMA, 0),
    ("long", MFMA, 512), ("long", VALU, 512), ("long", MFMA, 0),
    ("70b_fp8", MFMA, 0), ("70b_fp8", MFMA, 64), ("8b_fp8", MFMA, 0), ("8b_fp8", MFMA, 128),
    ("verify_fp8", MFMA, 0), ("long_fp8", MFMA, 512), ("long_fp8", MFMA, 0), ("d64_fp8", MFMA, 0),
]


@pytest.mark.parametrize("key,path,part", CASES, ids=[f"{k}-{'mfma' if p == 2 else 'valu'}-pt{t}" for k, p, t in CASES])
def test_parity_small(key, path, part):
    w, ref = small(key)
    print(f"case {key} path {path} part {part}", flush=True)
    out, _ = run_gpu(w, path=path, partition_tokens=part)
    assert_close(out_to_f64(out, w.cfg.dtype), ref, w.cfg.dtype, key)


SHAPES = [
    # dtype, q_len, H_q, H_kv, d, bs, context lengths
    ("bf16", 1, 8, 8, 64, 16, (5, 70, 300)),         # one query head per KV head, d 64
    ("bf16", 1, 16, 1, 64, 32, (31, 32, 33, 200)),   # 16 query heads on one KV head
    ("bf16", 4, 16, 2, 128, 32, (40, 129)),          # 8 x 4 = 32 rows: both row tiles full
    ("bf16", 2, 8, 2, 128, 16, (2, 17, 600)),        # context equal to q_len
    ("bf16", 8, 4, 1, 64, 16, (8, 9, 100)),          # 8 drafted tokens
    ("f32", 3, 4, 2, 128, 32, (3, 50, 301)),         # fp32 verification
    ("f32", 1, 16, 1, 128, 16, (1, 999)),            # fp32, 16 rows
    ("bf16", 1, 4, 2, 64, 32, (1, 64, 65)),          # bf16 d 64, block 32
]


def shape_cases():
    out = []
    for i, (dt, ql, hq, hkv, d, bs, lens) in enumerate(SHAPES):
        rows = hq // hkv * ql
        paths = ([MFMA] if dt == "bf16" and rows <= 32 else []) + ([VALU] if rows <= 16 else [])
        for path in paths:
            for pt in (0, 64):
                out.append((i, path, pt))
    return out


_shape_cache = {}


@pytest.mark.parametrize("i,path,pt", shape_cases(),
                         ids=[f"s{i}-{'mfma' if p == 2 else 'valu'}-pt{t}" for i, p, t in shape_cases()])
def test_parity_shapes(i, path, pt):
    if i not in _shape_cache:
        dt, ql, hq, hkv, d, bs, lens = SHAPES[i]
        cfg = workloads.Config(f"shape{i}", 100 + i, batch=len(lens), q_len=ql, num_q_heads=hq,
                               num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dt, lens=lens,
                               pool_slack=1.5)
        w = workloads.generate(cfg)
        _shape_cache[i] = (w, oracle_out(w))
    w, ref = _shape_cache[i]
    print(f"shape {SHAPES[i]} path {path} part {pt}", flush=True)
    out, _ = run_gpu(w, path=path, partition_tokens=pt)
    assert_close(out_to_f64(out, w.cfg.dtype), ref, w.cfg.dtype, f"shape {i}")


WAVE_CASES = [(k, wv) for k in ("8b", "70b", "verify", "long") for wv in (1, 2)]


@pytest.mark.parametrize("key,waves", WAVE_CASES, ids=[f"{k}-w{wv}" for k, wv in WAVE_CASES])
def test_parity_balanced_waves(key, waves):
    """The balanced schedule with 1 or 2 wavefronts per workgroup (grid and
    split points change with them)."""
    w, ref = small(key)
    out, _ = run_gpu(w, path=MFMA, waves=waves)
    assert_close(out_to_f64(out, w.cfg.dtype), ref, w.cfg.dtype, f"{key} waves {waves}")


@pytest.mark.parametrize("key", ["long", "8b", "verify"])
def test_balanced_repeat_calls_reuse_workspace(key):
    """Arrival counters are left zero, so repeated calls on one workspace give
    identical bits (a piece merged before all partials were visible would
    show up as a differing repeat)."""
    import paged_kv_cache_218_amd as pa
    w, ref = small(key)
    cfg = w.cfg
    out, cache = run_gpu(w, path=MFMA)
    desc = cache.desc(cfg.num_q_heads, int(w.lens.max()), MFMA, 0, 0)
    plan = pa.pa_attention_plan(desc, cfg.q_len)
    assert plan.schedule == pa.PA_SCHED_BALANCED
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    first = None
    for _ in range(8):
        o = torch.empty_like(out)
        q = torch.from_numpy(np.ascontiguousarray(w.q_all()).view(np.int16)).view(torch.bfloat16).cuda()
        pa.pa_attention(desc, q, cache.k_pool, cache.v_pool, cache.tables_device(),
                        torch.from_numpy(w.lens).cuda(), cfg.q_len, cfg.scale, o, ws)
        torch.cuda.synchronize()
        counters = ws[:cfg.batch * cfg.num_kv_heads * 4]
        assert int(counters.count_nonzero()) == 0
        if first is None:
            first = out_bits(o)
            assert_close(out_to_f64(o, "bf16"), ref, "bf16", f"repeat {key}")
        else:
            assert np.array_equal(out_bits(o), first)


@pytest.mark.parametrize("key", ["long", "8b"])
def test_schedules_share_one_workspace(key):
    """One cache, one workspace, calls alternating between schedules: the
    balanced schedule's arrival counters sit in an area no other schedule
    writes, so a balanced call after partition calls (whose partials fill the
    rest of the workspace) still merges its split sequences. Every call
    matches the oracle and leaves the counters zero."""
    import paged_kv_cache_218_amd as pa
    w, ref = small(key)
    cfg = w.cfg
    from paged_kv_cache_218_amd.cache import PagedKVCache
    cache = PagedKVCache.from_workload(w)
    seq = [(MFMA, 0), (MFMA, 128), (VALU, 64), (MFMA, 0), (MFMA, 64), (MFMA, 0)]
    scheds = []
    for path, pt in seq:
        print(f"{key}: path {path} partition_tokens {pt}", flush=True)
        out, _ = run_gpu(w, path=path, partition_tokens=pt, cache=cache)
        desc = cache.desc(cfg.num_q_heads, int(w.lens.max()), path, pt, 0)
        plan = pa.pa_attention_plan(desc, cfg.q_len)
        scheds.append(plan.schedule)
        assert_close(out_to_f64(out, cfg.dtype), ref, cfg.dtype, f"{key} path {path} pt {pt}")
        counters = cache._ws[:cfg.batch * cfg.num_kv_heads * 4]
        assert int(counters.count_nonzero()) == 0
    assert scheds.count(pa.PA_SCHED_BALANCED) == 3 and pa.PA_SCHED_PARTITIONS in scheds


@pytest.mark.parametrize("key", ["8b", "verify", "tiny_f32", "verify_fp8", "d64_fp8"])
def test_pool_bytes_and_tables_match_model(key):
    """pa_write_kv (allocation, copy-on-write, scatter, FP8 quantisation) gives
    the model's pool bit for bit."""
    w, _ = small(key)
    from paged_kv_cache_218_amd.cache import PagedKVCache
    import paged_kv_cache_218_amd as pa
    cache = PagedKVCache.from_workload(w)
    torch.cuda.synchronize()
    pool, model, tables, live = build_pool(w)
    assert np.array_equal(cache.tables, tables) and cache.live == live
    assert [pa.pa_block_refcount(cache.pool, b) for b in range(w.num_blocks)] == model.refcount
    assert list(pa.pa_pool_free_list(cache.pool)) == model.free_list()
    if w.cfg.kv_dtype == "fp8":
        codes = pool.k.size
        kb, vb = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
        assert np.array_equal(kb[:codes], pool.k.reshape(-1))
        assert np.array_equal(vb[:codes], pool.v.reshape(-1))
        assert np.array_equal(kb[codes:].view(np.uint32), pool.k_scale.reshape(-1).view(np.uint32))
        assert np.array_equal(vb[codes:].view(np.uint32), pool.v_scale.reshape(-1).view(np.uint32))
        return
    iview = torch.int32 if w.cfg.dtype == "f32" else torch.int16
    nview = np.int32 if w.cfg.dtype == "f32" else np.int16
    assert np.array_equal(cache.k_pool.cpu().view(iview).numpy(), pool.k.view(nview))
    assert np.array_equal(cache.v_pool.cpu().view(iview).numpy(), pool.v.view(nview))


def test_copy_blocks_bit_exact():
    w, _ = small("8b")
    from paged_kv_cache_218_amd.cache import PagedKVCache
    import paged_kv_cache_218_amd as pa
    cache = PagedKVCache.from_workload(w)
    k0, v0 = cache.k_pool.clone(), cache.v_pool.clone()
    used = [int(b) for b in cache.tables[0, :cache.live[0]]]
    free = list(pa.pa_pool_free_list(cache.pool))[:len(used)]
    pairs = np.array([[s, d] for s, d in zip(used, free)], dtype=np.int32)
    pa.pa_copy_blocks(cache.pool, cache.k_pool, cache.v_pool, pairs)
    torch.cuda.synchronize()
    for s, d in pairs:
        assert torch.equal(cache.k_pool[d].view(torch.int16), k0[s].view(torch.int16))
        assert torch.equal(cache.v_pool[d].view(torch.int16), v0[s].view(torch.int16))
    untouched = [b for b in range(w.num_blocks) if b not in set(pairs[:, 1].tolist())]
    assert torch.equal(cache.k_pool[untouched].view(torch.int16), k0[untouched].view(torch.int16))


@pytest.mark.parametrize("path", [MFMA, VALU])
def test_permuted_placement_bit_identical(path):
    w, _ = small("8b")
    a, _ = run_gpu(w, path=path)
    w2 = workloads.generate(workloads.config(*[SMALL["8b"][0]], **SMALL["8b"][1]))
    w2.free_order = np.random.default_rng(77).permutation(w2.num_blocks).astype(np.int32)
    b, c2 = run_gpu(w2, path=path)
    assert not np.array_equal(c2.tables, build_pool(w)[2])
    assert np.array_equal(out_bits(a), out_bits(b))


def test_shared_prefix_bit_identical_to_private_copies():
    w, _ = small("verify")
    w.num_blocks = w.cfg.batch * w.max_blocks
    w.free_order = workloads.free_order(w.cfg, w.num_blocks)
    a, ca = run_gpu(w, shared_prefix=True)
    b, cb = run_gpu(w, shared_prefix=False)
    assert np.array_equal(out_bits(a), out_bits(b))
    import paged_kv_cache_218_amd as pa
    assert pa.pa_pool_num_free(ca.pool) > pa.pa_pool_num_free(cb.pool)


@pytest.mark.parametrize("path", [MFMA, VALU])
def test_one_token_context_returns_v(path):
    cfg = workloads.config("llama3_70b_decode", batch=4, lens=(1, 1, 1, 1), len_const=0)
    w = workloads.generate(cfg)
    out, _ = run_gpu(w, path=path)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(4):
        want = np.repeat(w.seqs[b].v[0], cfg.group, axis=0)
        assert np.array_equal(got[b, 0], want)


def test_causal_rows_ignore_later_tokens():
    """Row i of a verification call must not see positions after L - q_len + i:
    overwrite those K/V slots with large values; earlier rows keep their bits."""
    w, _ = small("verify")
    cfg = w.cfg
    out1, cache = run_gpu(w)
    b, i = 2, 1
    L = int(w.lens[b])
    import paged_kv_cache_218_amd as pa
    n_after = L - (L - cfg.q_len + i + 1)
    big = torch.full((n_after, cfg.num_kv_heads, cfg.head_dim), 40.0, dtype=torch.bfloat16, device="cuda")
    cache.write(b, L - n_after, big, -big)
    out2, _ = run_gpu(w, cache=cache)
    o1, o2 = out_bits(out1), out_bits(out2)
    assert np.array_equal(o1[b, :i + 1], o2[b, :i + 1])
    assert not np.array_equal(o1[b, i + 1:], o2[b, i + 1:])
    others = [x for x in range(cfg.batch) if x != b]
    assert np.array_equal(o1[others], o2[others])


def test_verify_row_equals_decode_at_its_position():
    w, ref = small("verify")
    cfg = w.cfg
    out, cache = run_gpu(w)
    got = out_to_f64(out, "bf16")
    from paged_kv_cache_218_amd.cache import lens_to_device
    for i in range(cfg.q_len):
        q_i = torch.from_numpy(np.ascontiguousarray(w.q_all()[:, i:i + 1]).view(np.int16)).view(torch.bfloat16).cuda()
        lens_i = lens_to_device(w) - (cfg.q_len - 1 - i)
        o = cache.attention(q_i, cache.tables_device(), lens_i, 1, cfg.scale, int(w.lens.max()))
        torch.cuda.synchronize()
        assert_paths_agree(out_to_f64(o, "bf16")[:, 0], got[:, i], ref[:, i], "bf16", f"draft row {i} as a decode row")


def test_split_matches_unsplit():
    """Split-KV results do not depend on the partition size: every split meets
    the stated bar against the oracle."""
    w, ref = small("long")
    a, _ = run_gpu(w, partition_tokens=0)
    for pt in (64, 512, 2048):
        b, _ = run_gpu(w, partition_tokens=pt)
        assert_paths_agree(out_to_f64(a, "bf16"), out_to_f64(b, "bf16"), ref, "bf16", f"balanced vs partitions of {pt}")


def test_bad_lengths_and_tables_give_nan_not_faults():
    w, _ = small("8b")
    from paged_kv_cache_218_amd.cache import PagedKVCache, lens_to_device
    cache = PagedKVCache.from_workload(w)
    lens = lens_to_device(w)
    lens[1] = int(w.lens.max()) + 5        # beyond max_context
    lens[2] = 0                           # shorter than q_len
    tables = cache.tables_device()
    tables[3, 0] = w.num_blocks + 100     # block id outside the pool
    for path in (MFMA, VALU):
        for pt in (0, 128):
            out = cache.attention(torch.from_numpy(w.q_all().view(np.int16)).view(torch.bfloat16).cuda(),
                                  tables, lens, 1, w.cfg.scale, int(w.lens.max()), path=path, partition_tokens=pt)
            torch.cuda.synchronize()
            o = out_to_f64(out, "bf16")
            assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
            assert np.isfinite(o[[0, 4]]).all()
    # no valid sequence at all: nothing to split, every row NaN
    lens[:] = 0
    lens[0] = int(w.lens.max()) + 1
    for path in (MFMA, VALU):
        for pt in (0, 128):
            out = cache.attention(torch.from_numpy(w.q_all().view(np.int16)).view(torch.bfloat16).cuda(),
                                  tables, lens, 1, w.cfg.scale, int(w.lens.max()), path=path, partition_tokens=pt)
            torch.cuda.synchronize()
            assert np.isnan(out_to_f64(out, "bf16")).all(), (path, pt)


def _num_ranges(w, cache):
    """Ranges the balanced schedule cuts the (KV head, sequence, step) list
    into: min(grid, ceil(S / 8)), S = H_kv * sum of (ceil(L / 32) + segment
    cost) over the sequences (the plan's documented partition)."""
    import paged_kv_cache_218_amd as pa
    cfg = w.cfg
    pl = pa.pa_attention_plan(cache.desc(cfg.num_q_heads, int(w.lens.max()), MFMA), cfg.q_len)
    assert pl.schedule == pa.PA_SCHED_BALANCED and pl.segment_cost > 0
    units = sum(-(-int(L) // 32) + pl.segment_cost for L in w.lens)
    return min(pl.grid, -(-units * cfg.num_kv_heads // 8))


RANGE_CASES = [
    # (workload, overrides, whether the number of ranges is a multiple of 8, so
    # that each XCD takes consecutive ranges, i.e. whole KV heads)
    ("llama3_8b_decode", dict(batch=8, len_const=600), True),
    ("llama3_8b_decode", dict(batch=5, len_const=333), False),
    ("llama3_8b_decode", dict(batch=8, len_const=600, kv_dtype="fp8"), True),
    ("llama3_8b_decode", dict(batch=3, len_const=0, lens=(40, 333, 700), kv_dtype="fp8"), False),
    ("prefix_verify", dict(batch=8, prefix_len=64, len_lo=40, len_hi=500), None),
    ("tree_verify", dict(batch=6, prefix_len=32, len_lo=20, len_hi=400), None),
]


@pytest.mark.parametrize("name,kw,grouped", RANGE_CASES, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(RANGE_CASES)])
def test_balanced_range_to_workgroup_mapping(name, kw, grouped):
    """Ranges go to workgroups grouped by XCD when their number is a multiple
    of 8, one to one otherwise; both give the oracle's rows, and the batch's
    unit order (KV head major) covers every (sequence, KV head) exactly once."""
    from paged_kv_cache_218_amd.cache import PagedKVCache, tree_masks_to_device
    w = workloads.generate(workloads.config(name, **kw))
    cache = PagedKVCache.from_workload(w)
    n = _num_ranges(w, cache)
    print(f"{name} {kw}: {n} ranges", flush=True)
    if grouped is not None:
        assert (n % 8 == 0) == grouped, n
    tm = None if w.tree_parents is None else tree_masks_to_device(w.tree_parents)
    out, _ = run_gpu(w, path=MFMA, cache=cache, tree_mask=tm)
    if w.tree_parents is None:
        ref = oracle_out(w)
    else:
        rows = oracle_rows(w, range(w.cfg.batch))
        ref = np.stack([rows[b] for b in range(w.cfg.batch)])
    assert_close(out_to_f64(out, w.cfg.dtype), ref, w.cfg.dtype, f"{name} {n} ranges")
