"""Pins of the fp64 oracle against things other than itself (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import kvbytes, split
from oracle.build import build_pool
from oracle.numerics import to_f64
from oracle.store import HostPool
from tests.brute import brute_attention, brute_attention_logical

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(name, **kw):
    return workloads.generate(workloads.config(name, **kw))


SMALL = {
    "tiny_f32": dict(),
    "llama3_8b_decode": dict(batch=3, len_lo=40, len_hi=300),
    "llama3_70b_decode": dict(batch=2, len_const=200),
    "prefix_verify": dict(batch=4, prefix_len=40, len_lo=20, len_hi=70),
    "prefix_verify_aligned": None,
    "long_ctx_split": dict(batch=1, len_const=3000),
}


def small_workload(key):
    if key == "prefix_verify_aligned":
        return small("prefix_verify", batch=3, prefix_len=32, len_lo=16, len_hi=50)
    return small(key, **SMALL[key])


# -- input rounding ----------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, -1e-40,
                  np.inf, -np.inf], dtype=np.float32),
        # exact ties between two bf16 neighbours: mantissa bit pattern ...x8000
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = workloads.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # skip inf/nan patterns
    ours = to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# -- block tables printed on the pages --------------------------------------

@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "block_tables.json")))["cases"],
                         ids=lambda c: str(c["table"]))
def test_printed_block_tables(case):
    bs, n, table = case["block_size"], case["tokens"], case["table"]
    nb = max(table) + 1
    rng = np.random.default_rng(1)
    k = rng.standard_normal((n, 2, 32)).astype(np.float32)
    v = rng.standard_normal((n, 2, 32)).astype(np.float32)
    pool = HostPool(nb, bs, 2, 32, "f32")
    # place token p in physical block table[p // bs], slot p % bs, as the diagram draws it
    for p in range(n):
        pool.put_token(table[p // bs], p % bs, k[p], v[p])
    kg, vg = pool.gather(table, n)
    assert np.array_equal(kg, k) and np.array_equal(vg, v)
    # every other physical block is untouched (still NaN)
    others = [b for b in range(nb) if b not in table]
    assert np.isnan(pool.k[others]).all() and np.isnan(pool.v[others]).all()
    # the oracle sees the logical sequence: equal to attention on the unpaged arrays
    q = rng.standard_normal((1, 1, 4, 32)).astype(np.float32)
    out = oatt.attention_paged(q, pool, [table], [n], 1, 0.3)
    ref = oatt.attention_contiguous(q[0], k, v, 1, 4, 2, 0.3, "f32")
    assert np.array_equal(out[0], ref)


# -- brute force on tiny inputs ---------------------------------------------

@pytest.mark.parametrize("dtype,q_len,hq,hkv,d,bs,lens", [
    ("f32", 1, 4, 2, 32, 4, (1, 5, 9)),
    ("bf16", 1, 8, 2, 32, 4, (3, 8, 13)),
    ("f32", 3, 6, 3, 32, 2, (3, 7)),
    ("bf16", 4, 4, 1, 64, 8, (4, 11, 20)),
])
def test_oracle_vs_brute_force(dtype, q_len, hq, hkv, d, bs, lens):
    cfg = workloads.Config("brute", 90, batch=len(lens), q_len=q_len, num_q_heads=hq,
                           num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                           lens=lens, pool_slack=1.5)
    w = workloads.generate(cfg)
    pool, _, tables, _ = build_pool(w)
    got = oatt.attention_paged(w.q_all(), pool, tables, w.lens, q_len, 0.37)
    want = np.array(brute_attention(w.q_all(), pool.k, pool.v, tables, w.lens, q_len, 0.37, bs, dtype))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype,q_len,hq,hkv,d,bs,lens,prefix", [
    ("f32", 1, 4, 2, 32, 4, (1, 5, 9), 0),
    ("bf16", 3, 8, 2, 32, 4, (3, 8, 13), 0),
    ("bf16", 4, 4, 1, 64, 8, (4, 11, 20), 0),
    ("bf16", 2, 4, 2, 32, 4, (9, 14), 8),     # two blocks of a shared prefix
])
def test_oracle_vs_brute_force_on_never_paged_kv(dtype, q_len, hq, hkv, d, bs, lens, prefix):
    """The oracle's paged result against a scalar brute force over each
    sequence's K/V in token order, as the generator drew them: neither the
    pool's layout nor the block tables enter the reference side."""
    cfg = workloads.Config("brute", 91, batch=len(lens), q_len=q_len, num_q_heads=hq,
                           num_kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                           lens=lens, prefix_len=prefix, pool_slack=1.5)
    w = workloads.generate(cfg)
    pool, _, tables, _ = build_pool(w)
    got = oatt.attention_paged(w.q_all(), pool, tables, w.lens, q_len, 0.37)
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        assert k.shape[0] == w.lens[b]
        want = np.array(brute_attention_logical(w.seqs[b].q, k, v, q_len, 0.37, dtype))
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-13)


# -- torch's fp64 scaled_dot_product_attention on the never-paged K/V ------

def torch_sdpa_seq(q, k, v, q_len, G, scale, dtype, kv_dtype=None):
    kvd = kv_dtype or dtype
    conv = (lambda a: np.asarray(a, dtype=np.float64)) if kvd == "f64" else (lambda a: to_f64(a, kvd))
    qt = torch.from_numpy(to_f64(q, dtype)).permute(1, 0, 2)[None]          # [1,Hq,q,d]
    kt = torch.from_numpy(conv(k)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(conv(v)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    L = k.shape[0]
    mask = torch.ones(q_len, L, dtype=torch.bool).tril(diagonal=L - q_len)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("key", list(SMALL))
def test_oracle_vs_torch_sdpa(key):
    w = small_workload(key)
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    got = oatt.attention_paged(w.q_all(), pool, tables, w.lens, cfg.q_len, cfg.scale)
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        ref = torch_sdpa_seq(w.seqs[b].q, k, v, cfg.q_len, cfg.group, cfg.scale, cfg.dtype)
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)


# -- invariants --------------------------------------------------------------

def test_permuted_placement_is_bit_identical():
    w = small_workload("llama3_8b_decode")
    pool, _, tables, _ = build_pool(w)
    ref = oatt.attention_paged(w.q_all(), pool, tables, w.lens, 1, w.cfg.scale)
    for seed in (5, 6):
        w2 = small_workload("llama3_8b_decode")
        w2.free_order = np.random.default_rng(seed).permutation(w2.num_blocks).astype(np.int32)
        pool2, _, tables2, _ = build_pool(w2)
        assert not np.array_equal(tables, tables2)
        out = oatt.attention_paged(w2.q_all(), pool2, tables2, w2.lens, 1, w2.cfg.scale)
        assert np.array_equal(out, ref)


@pytest.mark.parametrize("key", ["prefix_verify", "prefix_verify_aligned"])
def test_shared_prefix_equals_private_copies(key):
    w = small_workload(key)
    # room for a private prefix copy per sequence
    w.num_blocks = w.cfg.batch * w.max_blocks
    w.free_order = workloads.free_order(w.cfg, w.num_blocks)
    pool_s, model_s, tab_s, _ = build_pool(w, shared_prefix=True)
    pool_p, model_p, tab_p, _ = build_pool(w, shared_prefix=False)
    a = oatt.attention_paged(w.q_all(), pool_s, tab_s, w.lens, w.cfg.q_len, w.cfg.scale)
    b = oatt.attention_paged(w.q_all(), pool_p, tab_p, w.lens, w.cfg.q_len, w.cfg.scale)
    assert np.array_equal(a, b)
    assert model_s.num_free > model_p.num_free       # sharing saved blocks


def test_one_token_context_returns_v_exactly():
    cfg = workloads.config("llama3_70b_decode", batch=3, lens=(1, 1, 1), len_const=0)
    w = workloads.generate(cfg)
    pool, _, tables, _ = build_pool(w)
    out = oatt.attention_paged(w.q_all(), pool, tables, w.lens, 1, cfg.scale)
    for b in range(3):
        v = to_f64(w.seqs[b].v[0], "bf16")                       # [H_kv][d]
        assert np.array_equal(out[b, 0], np.repeat(v, cfg.group, axis=0))


def test_zero_query_gives_mean_of_values():
    w = small_workload("llama3_8b_decode")
    for s in w.seqs:
        s.q[:] = 0
    pool, _, tables, _ = build_pool(w)
    out = oatt.attention_paged(w.q_all(), pool, tables, w.lens, 1, w.cfg.scale)
    for b in range(w.cfg.batch):
        _, v = w.logical_kv(b)
        mean = to_f64(v, "bf16").mean(axis=0)                    # [H_kv][d]
        np.testing.assert_allclose(out[b, 0], np.repeat(mean, w.cfg.group, axis=0), rtol=0, atol=1e-14)


def test_causal_rows():
    w = small_workload("prefix_verify")
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    out = oatt.attention_paged(w.q_all(), pool, tables, w.lens, cfg.q_len, cfg.scale)
    b = 1
    L = int(w.lens[b])
    for i in range(cfg.q_len):
        # row i equals a one-row call on the context that ends at its own position
        single = oatt.attention_paged_seq(w.seqs[b].q[i:i + 1], pool, tables[b], L - cfg.q_len + i + 1,
                                          1, cfg.num_q_heads, cfg.scale)
        assert np.array_equal(single[0], out[b, i])
    # perturbing keys/values after row i's position leaves row i unchanged
    pert = HostPool(pool.nb, pool.bs, pool.hkv, pool.d, pool.dtype)
    pert.k[:], pert.v[:] = pool.k, pool.v
    i = 1
    for t in range(L - cfg.q_len + i + 1, L):
        blk, off = tables[b][t // cfg.block_size], t % cfg.block_size
        pert.put_token(blk, off,
                       workloads.bf16_bits_from_f32(np.full((cfg.num_kv_heads, cfg.head_dim), 50.0, np.float32)),
                       workloads.bf16_bits_from_f32(np.full((cfg.num_kv_heads, cfg.head_dim), -7.0, np.float32)))
    out2 = oatt.attention_paged_seq(w.seqs[b].q, pert, tables[b], L, cfg.q_len, cfg.num_q_heads, cfg.scale)
    assert np.array_equal(out2[:i + 1], out[b, :i + 1])
    assert not np.allclose(out2[i + 1:], out[b, i + 1:])


# -- split-KV identity ---------------------------------------------------------

@pytest.mark.parametrize("part", [128, 512, 4096])
def test_split_merge_equals_direct(part):
    w = small_workload("long_ctx_split")
    cfg = w.cfg
    k, v = w.logical_kv(0)
    q = to_f64(w.seqs[0].q[0], "bf16")
    for g in (0, 5):
        kf, vf = to_f64(k[:, g], "bf16"), to_f64(v[:, g], "bf16")
        rows = q[g * cfg.group:(g + 1) * cfg.group]
        direct = oatt.attend(rows, kf, vf, cfg.scale)
        merged = split.attend_split(rows, kf, vf, cfg.scale, part)
        np.testing.assert_allclose(merged, direct, rtol=1e-12, atol=1e-15)


def test_merge_of_single_partition_is_identity():
    rng = np.random.default_rng(3)
    m, l, o = rng.standard_normal((1, 4)), rng.random((1, 4)) + 0.5, rng.standard_normal((1, 4, 16))
    np.testing.assert_allclose(split.lse_merge(m, l, o), o[0], rtol=1e-15)


def test_merge_survives_far_apart_maxima():
    # two partitions whose maxima differ by 1000: the small one must vanish, no overflow
    m = np.array([[1000.0], [0.0]])
    l = np.array([[2.0], [3.0]])
    o = np.array([[[1.0, 2.0]], [[5.0, 6.0]]])
    np.testing.assert_allclose(split.lse_merge(m, l, o), [[1.0, 2.0]], rtol=1e-15)


# -- closed form for KV bytes -----------------------------------------------

@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))["cases"],
                         ids=lambda c: f"L{c['num_layers']}xS{c['seq_len']}")
def test_kv_bytes_closed_form(case):
    got = kvbytes.kv_bytes(case["num_layers"], case["num_kv_heads"], case["head_dim"],
                           case["elem_bytes"], case["seq_len"])
    assert got == case["bytes"]
    # 4 * L * H_kv * d_k per token at 16-bit storage
    assert got == 4 * case["num_layers"] * case["num_kv_heads"] * case["head_dim"] * case["seq_len"]
    if "printed_mib_thousands" in case:
        assert math.isclose(got / 2**20 / 1000, case["printed_mib_thousands"], rel_tol=1e-3)
    if "page_double_counted_bytes" in case:
        assert 2 * got == case["page_double_counted_bytes"]


def test_kv_bytes_of_the_70b_decode_workload():
    cfg = workloads.CONFIGS["llama3_70b_decode"]
    per_layer = kvbytes.kv_bytes_per_token(1, cfg.num_kv_heads, cfg.head_dim, 2)
    assert per_layer == 4096
    pool_bytes = 16384 * cfg.block_size * per_layer
    assert pool_bytes == 2**31
    # one layer's share of the 64 x 8192-token example
    assert pool_bytes * 80 == kvbytes.kv_bytes(80, 8, 128, 2, 64 * 8192)
