"""Tree-structured verification on the HIP path vs the fp64 oracle (MI355X).

Masks reach the device from the library's own pa_tree_masks; the oracle
builds its ancestor sets from the same parent indices on its own."""
import numpy as np
import pytest

import workloads
from oracle import tree as otree
from oracle.build import build_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import assert_close, out_bits, out_to_f64, run_gpu  # noqa: E402

VALU, MFMA = 1, 2

TREES = {
    # 4 query heads per KV head x 8 nodes = 32 rows (two MFMA row tiles)
    "tree8": ("tree_verify", dict(batch=6, prefix_len=40, len_lo=20, len_hi=300)),
    "tree8_shared": ("tree_verify", dict(batch=5, prefix_len=40, len_lo=5, len_hi=200, tree="shared")),
    # 3 nodes x 4 heads = 12 rows (one row tile); a context of exactly the drafted tokens
    "tree3": ("tree_verify", dict(batch=4, q_len=3, prefix_len=0, len_lo=0, len_hi=0, lens=(3, 4, 50, 333))),
    # one query head per KV head and 32 nodes: every mask bit in use
    "tree32": ("tree_verify", dict(batch=3, q_len=32, num_q_heads=2, num_kv_heads=2, head_dim=64, prefix_len=0,
                                   len_lo=0, len_hi=0, lens=(32, 45, 200))),
    "tree8_fp8": ("tree_verify", dict(batch=6, prefix_len=40, len_lo=20, len_hi=300, kv_dtype="fp8")),
    "tree4_f32": ("tree_verify", dict(batch=4, q_len=4, dtype="f32", prefix_len=16, len_lo=1, len_hi=100)),
    "tree6_70b": ("tree_verify", dict(batch=3, q_len=4, num_q_heads=64, num_kv_heads=8, block_size=32,
                                      prefix_len=0, len_lo=100, len_hi=700)),
}
_cache = {}


def tree_case(key):
    if key not in _cache:
        name, kw = TREES[key]
        w = workloads.generate(workloads.config(name, **kw))
        masks = [otree.ancestor_masks(p) for p in w.tree_parents]
        pool, _, tables, _ = build_pool(w)
        ref = otree.attention_tree(w.q_all(), pool, tables, w.lens, w.cfg.q_len, masks, w.cfg.scale)
        _cache[key] = (w, ref)
    return _cache[key]


def device_masks(w):
    from paged_kv_cache_218_amd.cache import tree_masks_to_device
    return tree_masks_to_device(w.tree_parents)


CASES = [("tree8", MFMA, 0), ("tree8", MFMA, 64), ("tree8_shared", MFMA, 0), ("tree3", MFMA, 0),
         ("tree3", VALU, 0), ("tree3", MFMA, 128), ("tree32", MFMA, 0), ("tree32", MFMA, 64),
         ("tree8_fp8", MFMA, 0), ("tree8_fp8", MFMA, 64), ("tree4_f32", VALU, 0), ("tree4_f32", VALU, 64),
         ("tree6_70b", MFMA, 0)]


@pytest.mark.parametrize("key,path,part", CASES,
                         ids=[f"{k}-{'mfma' if p == 2 else 'valu'}-pt{t}" for k, p, t in CASES])
def test_tree_parity(key, path, part):
    w, ref = tree_case(key)
    print(f"tree case {key} path {path} part {part}", flush=True)
    out, _ = run_gpu(w, path=path, partition_tokens=part, tree_mask=device_masks(w))
    assert_close(out_to_f64(out, w.cfg.dtype), ref, w.cfg.dtype, key)


def test_shared_mask_stride_zero_equals_per_sequence():
    w, ref = tree_case("tree8_shared")
    masks = device_masks(w)
    print("tree shared masks, stride 0", flush=True)
    per_seq, cache = run_gpu(w, path=MFMA, tree_mask=masks)
    one = masks[0].contiguous()
    shared, _ = run_gpu(w, path=MFMA, cache=cache, tree_mask=one, mask_stride=0)
    assert np.array_equal(out_bits(per_seq), out_bits(shared))


@pytest.mark.parametrize("path,part", [(MFMA, 0), (MFMA, 64), (VALU, 0)])
def test_chain_masks_bit_identical_to_causal(path, part):
    """A chain of drafted tokens is plain verification: the tree entry point
    with chain masks gives the causal entry point's bits."""
    name, kw = TREES["tree3"]
    w = workloads.generate(workloads.config(name, **kw))
    chain = np.tile(np.arange(-1, w.cfg.q_len - 1, dtype=np.int32), (w.cfg.batch, 1))
    from paged_kv_cache_218_amd.cache import tree_masks_to_device
    print(f"tree chain vs causal path {path} part {part}", flush=True)
    causal, cache = run_gpu(w, path=path, partition_tokens=part)
    tree, _ = run_gpu(w, path=path, partition_tokens=part, cache=cache, tree_mask=tree_masks_to_device(chain))
    assert np.array_equal(out_bits(causal), out_bits(tree))


@pytest.mark.parametrize("path", [MFMA, VALU])
def test_arbitrary_masks_self_bit_and_high_bits(path):
    """Any 32-bit mask is accepted: the row's own bit counts as set and bits at
    or past q_len are ignored (random masks, not ancestor sets)."""
    name, kw = TREES["tree3"]
    w = workloads.generate(workloads.config(name, **kw))
    cfg = w.cfg
    rng = np.random.default_rng(31)
    masks = rng.integers(0, 2**32, size=(cfg.batch, cfg.q_len), dtype=np.uint64).astype(np.uint32)
    masks[0, :] = 0                       # nothing but itself
    pool, _, tables, _ = build_pool(w)
    ref = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks.tolist(), cfg.scale)
    dev = torch.from_numpy(masks.view(np.int32).copy()).cuda()
    print(f"tree random masks path {path}", flush=True)
    out, _ = run_gpu(w, path=path, tree_mask=dev)
    assert_close(out_to_f64(out, cfg.dtype), ref, cfg.dtype, "random masks")


def test_tree_rows_ignore_other_branches():
    """Overwriting the K/V of one node changes exactly the rows that see it."""
    w, _ = tree_case("tree8_shared")
    cfg = w.cfg
    masks_dev = device_masks(w)
    base, cache = run_gpu(w, path=MFMA, tree_mask=masks_dev)
    masks = [otree.ancestor_masks(p) for p in w.tree_parents]
    j = int(np.argmax([bin(m).count("1") for m in masks[0]]))   # a node deep in the tree
    node = int(w.tree_parents[0][j])
    node = j if node < 0 else node
    k_new = torch.full((1, cfg.num_kv_heads, cfg.head_dim), 2.5, dtype=torch.bfloat16, device="cuda")
    # rewrite that node's K in place in every sequence (positions L - q_len + node)
    for b in range(cfg.batch):
        pos = int(w.lens[b]) - cfg.q_len + node
        cache.write(b, pos, k_new, k_new)
    print(f"tree node {node} overwritten", flush=True)
    out, _ = run_gpu(w, path=MFMA, cache=cache, tree_mask=masks_dev)
    a, o = out_bits(base), out_bits(out)
    for b in range(cfg.batch):
        for i in range(cfg.q_len):
            sees = bool((masks[b][i] >> node) & 1)
            assert (not np.array_equal(a[b, i], o[b, i])) == sees, (b, i, node)
