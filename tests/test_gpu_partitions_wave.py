"""Fixed partitions with one wavefront per partition (PA_SCHED_PARTITIONS_WAVE)
against the fp64 oracle through the C ABI: decode at block sizes 16 and 32,
lengths on either side of partition edges (sequences of one partition write
their rows directly, longer ones go through the merge kernel), causal and
tree verification (two row tiles), FP8 pools, head dim 64, and bad lengths or
block ids, which give NaN rows. Every case is sized so that the plan picks
the per-wave kernel (the partitions alone fill the device's wave slots)."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import assert_close, oracle_rows, out_to_f64, run_gpu  # noqa: E402

# 32 lengths around the edges of 64-token partitions and 16/32-token blocks
EDGES = (1, 17, 63, 64, 65, 128, 129, 500, 1000, 1500, 2047, 2048, 2049, 2500, 3000, 3001) * 2

CASES = {
    "decode_bs32": ("llama3_70b_decode", dict(batch=4, len_const=8192)),
    "decode_edges": ("llama3_8b_decode", dict(batch=32, len_const=0, lens=EDGES)),
    "verify": ("prefix_verify", dict(batch=16, prefix_len=40, len_lo=1000, len_hi=2000)),
    "tree": ("tree_verify", dict(batch=16, prefix_len=40, len_lo=1000, len_hi=2000)),
    "decode_fp8": ("llama3_70b_decode_fp8", dict(batch=8, len_const=4096)),
    "verify_fp8": ("prefix_verify", dict(batch=16, prefix_len=40, len_lo=1000, len_hi=2000, kv_dtype="fp8")),
    "d64": ("llama3_70b_decode", dict(batch=32, len_const=0, lens=EDGES, head_dim=64, num_q_heads=16,
                                      num_kv_heads=4)),
}
PT = 64


def plan_of(cache, w, pt):
    import paged_kv_cache_218_amd as pa
    return pa.pa_attention_plan(cache.desc(w.cfg.num_q_heads, int(w.lens.max()), 0, pt), w.cfg.q_len)


@pytest.mark.parametrize("key", list(CASES))
def test_per_wave_partitions_match_oracle(key):
    import paged_kv_cache_218_amd as pa
    name, kw = CASES[key]
    w = workloads.generate(workloads.config(name, **kw))
    print(f"case {key}", flush=True)
    masks = None
    if w.tree_parents is not None:
        from paged_kv_cache_218_amd.cache import tree_masks_to_device
        masks = tree_masks_to_device(w.tree_parents)
    out, cache = run_gpu(w, partition_tokens=PT, tree_mask=masks)
    plan = plan_of(cache, w, PT)
    assert plan.schedule == pa.PA_SCHED_PARTITIONS_WAVE and plan.merge_grid > 0
    got = out_to_f64(out, w.cfg.dtype)
    ref = oracle_rows(w, range(w.cfg.batch))
    for b in range(w.cfg.batch):
        assert_close(got[b], ref[b], w.cfg.dtype, f"{key} seq {b} (L={w.lens[b]})")


def test_per_wave_partitions_bad_lengths_and_tables_give_nan():
    import paged_kv_cache_218_amd as pa
    from paged_kv_cache_218_amd.cache import PagedKVCache, lens_to_device, queries_to_device
    name, kw = CASES["decode_edges"]
    w = workloads.generate(workloads.config(name, **kw))
    cache = PagedKVCache.from_workload(w)
    assert plan_of(cache, w, PT).schedule == pa.PA_SCHED_PARTITIONS_WAVE
    lens = lens_to_device(w)
    lens[9] = int(w.lens.max()) + 5        # beyond max_context
    lens[10] = 0                          # shorter than q_len
    tables = cache.tables_device()
    tables[11, 3] = w.num_blocks + 100    # block id outside the pool (a sequence of 2047 tokens)
    tables[2, 0] = -7                     # the only block of a one-partition sequence (63 tokens)
    out = cache.attention(queries_to_device(w), tables, lens, 1, w.cfg.scale, int(w.lens.max()),
                          partition_tokens=PT)
    torch.cuda.synchronize()
    o = out_to_f64(out, "bf16")
    for b in (2, 9, 10, 11):
        assert np.isnan(o[b]).all(), b
    good = [b for b in range(w.cfg.batch) if b not in (2, 9, 10, 11)]
    assert np.isfinite(o[good]).all()
    ref = oracle_rows(w, good)
    for b in good:
        assert_close(o[b], ref[b], "bf16", f"seq {b}")


def test_runs_bit_identical_to_one_partition_per_wave():
    """With more partitions than wave slots, each wavefront streams a run of
    consecutive partitions (parking the finished ones' states in LDS); every
    partition is still computed on its own, so the rows equal, bit for bit,
    those of a batch whose partitions exactly fill the wave slots (one
    partition per wavefront), and match the oracle."""
    import paged_kv_cache_218_amd as pa
    from tests.gpu_util import out_bits
    base = workloads.config("llama3_70b_decode", batch=4, len_const=0, lens=(8192, 8192 - 37, 8000, 8192))
    w4 = workloads.generate(base)
    w3 = workloads.generate(workloads.config("llama3_70b_decode", batch=3, len_const=0,
                                             lens=(8192, 8192 - 37, 8000)))
    out4, cache4 = run_gpu(w4, partition_tokens=PT)
    out3, cache3 = run_gpu(w3, partition_tokens=PT)
    p4, p3 = plan_of(cache4, w4, PT), plan_of(cache3, w3, PT)
    assert p4.schedule == pa.PA_SCHED_PARTITIONS_WAVE and p4.partitions_per_wave > 1
    if p3.schedule != pa.PA_SCHED_PARTITIONS_WAVE or p3.partitions_per_wave != 1:
        pytest.skip("the three-sequence batch does not exactly fill this device's wave slots")
    # the two batches' sequences 0-2 are the same seeded data only if the generator draws them alike
    assert np.array_equal(w4.q_all()[:3], w3.q_all())
    b4, b3 = out_bits(out4), out_bits(out3)
    assert np.array_equal(b4[:3], b3)
    got = out_to_f64(out4, "bf16")
    ref = oracle_rows(w4, range(4))
    for b in range(4):
        assert_close(got[b], ref[b], "bf16", f"runs seq {b}")
