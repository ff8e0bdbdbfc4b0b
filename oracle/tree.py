"""Tree-structured speculative verification in float64. TEST INFRASTRUCTURE ONLY.

Page "Mở rộng Quy mô và Triển khai", section "Giải mã Suy đoán (Speculative
Decoding)", its list of variants: parallel decoding drafts several
continuations at once, a tree of candidate tokens, and the target verifies the
whole tree in one pass. The pages print no mask. Readings taken here:
  * the q_len tree nodes are the last q_len positions of the sequence: node j
    sits at position L - q_len + j, its K/V written there before the call;
  * parent[j] is the node that j continues (parent[j] < j), or -1 when j
    continues the context's last token directly;
  * node i sees the whole context (positions 0 .. L - q_len - 1) and the
    nodes on its path to the root, itself included (its ancestor set). With
    parent[j] = j - 1 for every node this is the causal triangle of plain
    verification;
  * a caller may pass any visibility bitmask per node (bit j: sees node j);
    bit i of node i is always taken as set, so no row is empty, and bits at
    or above q_len name no node and are ignored.
The attention itself is the definition used everywhere else
(softmax(q K^T * scale) V) over the visible positions only.
"""
from __future__ import annotations

import numpy as np

from .attention import _q_dtype, attend
from .numerics import to_f64
from .store import HostPool

MAX_NODES = 32  # one 32-bit mask per node


def ancestor_masks(parents) -> list:
    """Bit j of masks[i] is set iff node j is node i or one of its ancestors."""
    n = len(parents)
    if n > MAX_NODES:
        raise ValueError("at most 32 tree nodes")
    masks = []
    for i, p in enumerate(parents):
        p = int(p)
        if not (p == -1 or 0 <= p < i):
            raise ValueError(f"parent of node {i} must be -1 or an earlier node, got {p}")
        masks.append((1 << i) | (masks[p] if p >= 0 else 0))
    return masks


def visible_positions(L: int, q_len: int, mask: int, i: int) -> np.ndarray:
    """Positions that node i of a q_len-node tree at the end of an L-token
    sequence sees: the context, then the nodes whose bit is set."""
    ctx = L - q_len
    bits = (int(mask) | (1 << i)) & ((1 << q_len) - 1)
    nodes = [j for j in range(q_len) if (bits >> j) & 1]
    return np.concatenate([np.arange(ctx, dtype=np.int64), ctx + np.asarray(nodes, dtype=np.int64)])


def attention_tree_seq(q, pool: HostPool, table, ctx_len: int, q_len: int, masks,
                       num_q_heads: int, scale: float, q_dtype: str = None) -> np.ndarray:
    """One sequence: q [q_len][H_q][d], masks [q_len] (ints). float64 out."""
    G = num_q_heads // pool.hkv
    qf = to_f64(q, _q_dtype(pool, q_dtype))
    out = np.empty(qf.shape, dtype=np.float64)
    for g in range(pool.hkv):
        kf, vf = pool.gather_head_f64(table, ctx_len, g)
        for i in range(q_len):
            pos = visible_positions(ctx_len, q_len, masks[i], i)
            rows = qf[i, g * G:(g + 1) * G, :]
            out[i, g * G:(g + 1) * G, :] = attend(rows, kf[pos], vf[pos], scale)
    return out


def attention_tree_contiguous(q, k, v, q_len: int, num_q_heads: int, num_kv_heads: int, masks,
                              scale: float, dtype: str, kv_dtype: str = None) -> np.ndarray:
    """One sequence with contiguous (never-paged) K/V [L][H_kv][d]; masks [q_len]."""
    G = num_q_heads // num_kv_heads
    L = k.shape[0]
    qf = to_f64(q, dtype)
    out = np.empty(qf.shape, dtype=np.float64)
    for g in range(num_kv_heads):
        kf = to_f64(k[:, g, :], kv_dtype or dtype)
        vf = to_f64(v[:, g, :], kv_dtype or dtype)
        for i in range(q_len):
            pos = visible_positions(L, q_len, masks[i], i)
            out[i, g * G:(g + 1) * G, :] = attend(qf[i, g * G:(g + 1) * G, :], kf[pos], vf[pos], scale)
    return out


def attention_tree(q, pool: HostPool, tables, ctx_lens, q_len: int, masks, scale: float,
                   q_dtype: str = None) -> np.ndarray:
    """Batch form. q [B][q_len][H_q][d]; masks [B][q_len]. float64 out."""
    B, _, Hq, _ = q.shape
    return np.stack([attention_tree_seq(q[b], pool, tables[b], int(ctx_lens[b]), q_len,
                                        [int(m) for m in masks[b]], Hq, scale, q_dtype)
                     for b in range(B)])
