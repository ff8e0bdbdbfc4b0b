"""Pins of the tree-verification oracle (CPU only).

The oracle builds visibility from ancestor bitmasks; the pins below build it
other ways: by walking parent pointers into a boolean mask for torch's fp64
scaled_dot_product_attention, by a scalar brute force over the root path,
and by the special trees whose answer is already pinned elsewhere (a chain is
plain causal verification).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import tree as otree
from oracle.build import build_pool
from oracle.numerics import to_f64
from tests.brute import scalar


def tree_workload(**kw):
    base = dict(batch=3, prefix_len=24, len_lo=20, len_hi=60)
    base.update(kw)
    return workloads.generate(workloads.config("tree_verify", **base))


def path_to_root(parents, i):
    out = []
    while i >= 0:
        out.append(i)
        i = int(parents[i])
    return out


def masks_of(w):
    return [otree.ancestor_masks(p) for p in w.tree_parents]


def test_ancestor_masks_literal():
    # node 0 and node 4 continue the context; 1, 2 hang off 0; 3 off 1
    assert otree.ancestor_masks([-1, 0, 0, 1, -1]) == [0b00001, 0b00011, 0b00101, 0b01011, 0b10000]
    assert otree.ancestor_masks([-1, 0, 1, 2]) == [0b1, 0b11, 0b111, 0b1111]    # chain: causal
    assert otree.ancestor_masks([-1] * 4) == [1, 2, 4, 8]                        # star
    with pytest.raises(ValueError):
        otree.ancestor_masks([-1, 1])        # a node cannot be its own parent
    with pytest.raises(ValueError):
        otree.ancestor_masks([-1] * 33)      # one 32-bit mask per node


def test_visible_positions_rules():
    # L = 10, 4 nodes at positions 6..9; node 2 with mask 0b0101 sees 0..5, 6, 8
    assert otree.visible_positions(10, 4, 0b0101, 2).tolist() == [0, 1, 2, 3, 4, 5, 6, 8]
    # its own bit is always set; bits past the last node are ignored
    assert otree.visible_positions(10, 4, 0, 3).tolist() == [0, 1, 2, 3, 4, 5, 9]
    assert otree.visible_positions(10, 4, 0b1 | (1 << 31), 0).tolist() == [0, 1, 2, 3, 4, 5, 6]


def test_chain_tree_equals_causal_verification():
    w = tree_workload()
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    chain = [otree.ancestor_masks(list(range(-1, cfg.q_len - 1)))] * cfg.batch
    got = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, chain, cfg.scale)
    ref = oatt.attention_paged(w.q_all(), pool, tables, w.lens, cfg.q_len, cfg.scale)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kw", [dict(), dict(tree="shared"), dict(q_len=5, lens=(5, 6, 40), prefix_len=0,
                                                                   len_lo=0, len_hi=0)])
def test_tree_vs_torch_sdpa_with_parent_walk_mask(kw):
    w = tree_workload(**kw)
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    got = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks_of(w), cfg.scale)
    G = cfg.group
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        L = k.shape[0]
        ctx = L - cfg.q_len
        mask = torch.zeros(cfg.q_len, L, dtype=torch.bool)
        mask[:, :ctx] = True
        for i in range(cfg.q_len):
            for j in path_to_root(w.tree_parents[b], i):
                mask[i, ctx + j] = True
        qt = torch.from_numpy(to_f64(w.seqs[b].q, "bf16")).permute(1, 0, 2)[None]
        kt = torch.from_numpy(to_f64(k, "bf16")).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(to_f64(v, "bf16")).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=cfg.scale)
        np.testing.assert_allclose(got[b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_tree_row_vs_scalar_brute_force_over_root_path():
    w = tree_workload(batch=2, q_len=6, num_q_heads=4, num_kv_heads=2, head_dim=32, prefix_len=5,
                      len_lo=3, len_hi=12)
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    got = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks_of(w), cfg.scale)
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        L = k.shape[0]
        for i in range(cfg.q_len):
            # attention over a set is order-free: context then the root path, leaf first
            pos = list(range(L - cfg.q_len)) + [L - cfg.q_len + j for j in path_to_root(w.tree_parents[b], i)]
            for h in range(cfg.num_q_heads):
                g = h // cfg.group
                qv = [scalar(x, "bf16") for x in w.seqs[b].q[i, h]]
                sc = [cfg.scale * math.fsum(qv[c] * scalar(k[t, g, c], "bf16") for c in range(cfg.head_dim))
                      for t in pos]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = math.fsum(e)
                for c in range(cfg.head_dim):
                    ref = math.fsum(e[n] * scalar(v[t, g, c], "bf16") for n, t in enumerate(pos)) / z
                    assert abs(got[b, i, h, c] - ref) <= 1e-13


def test_tree_rows_independent_of_other_branches():
    # perturbing the K/V of node j changes exactly the rows whose ancestor set holds j
    w = tree_workload(batch=1, tree="shared")
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    masks = masks_of(w)
    base = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks, cfg.scale)
    L = int(w.lens[0])
    for j in range(cfg.q_len):
        pos = L - cfg.q_len + j
        blk, off = tables[0][pos // cfg.block_size], pos % cfg.block_size
        saved = pool.k[blk].copy()
        pool.k[blk, :, :, off, :] = workloads.bf16_bits_from_f32(np.full(pool.k[blk, :, :, off, :].shape, 3.0,
                                                                         np.float32))
        out = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks, cfg.scale)
        pool.k[blk] = saved
        for i in range(cfg.q_len):
            changed = not np.array_equal(out[0, i], base[0, i])
            assert changed == bool((masks[0][i] >> j) & 1), (i, j)


def test_contiguous_form_equals_paged_form():
    w = tree_workload()
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    masks = masks_of(w)
    paged = otree.attention_tree(w.q_all(), pool, tables, w.lens, cfg.q_len, masks, cfg.scale)
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        flat = otree.attention_tree_contiguous(w.seqs[b].q, k, v, cfg.q_len, cfg.num_q_heads, cfg.num_kv_heads,
                                               masks[b], cfg.scale, cfg.dtype)
        assert np.array_equal(flat, paged[b])
