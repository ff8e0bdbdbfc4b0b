"""Reference paged attention in float64.

Definition (Part 8, section "Thực Thi Kernel Toán Học Trong CUDA"): for a
query vector q_i and the keys K of its context, the attention weights are
softmax(q_i K^T / sqrt(d_k)) and the output is the weighted sum of the value
vectors. Under paging the keys and values of a sequence are spread over
physical blocks B_1..B_m and the kernel walks them block by block; its output
sums a_{i,j,t} v_{(j,t)} over every block j and every slot t. The pages do not
define a_{i,j,t}; the reading taken here is the plain one: a is the softmax
over all (j, t) of the concatenated block scores, i.e. exactly the unpaged
definition on the gathered context. The oracle therefore gathers each
sequence's contiguous K/V through its block table and applies the unpaged
formula; the block-by-block online softmax is the kernel's business.

Readings of points the pages leave open:
  * GQA grouping (Blog #54, section 4 and Part 8's Llama-3-70B example name 8
    KV heads shared by the query heads): query head h reads KV head h // G with
    G = H_q / H_kv (contiguous groups).
  * scale is passed in; the workloads use 1/sqrt(d).
  * Several query rows per sequence (speculative verification: the target
    runs one pass over the context followed by the drafted tokens; Part 8,
    "Speculative Decoding" sequence diagram; Blog #54, section 2.4): the
    context length L counts the drafted tokens, which sit at the last q_len
    positions, and row i (0-based) sees positions 0 .. L - q_len + i.
"""
from __future__ import annotations

import numpy as np

from .numerics import to_f64
from .store import HostPool


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax of a 2-D float64 score array."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for query rows q [R][d] over K, V [T][d] (fp64)."""
    return softmax_rows(scale * (q @ k.T)) @ v


def attention_contiguous(q, k, v, q_len: int, num_q_heads: int, num_kv_heads: int,
                         scale: float, dtype: str, kv_dtype: str = None) -> np.ndarray:
    """One sequence with contiguous K/V.

    q: [q_len][H_q][d]; k, v: [L][H_kv][d] in storage format (kv_dtype, default
    dtype; "f64" for values already in float64, e.g. dequantised FP8).
    Returns float64 [q_len][H_q][d].
    """
    G = num_q_heads // num_kv_heads
    L = k.shape[0]
    qf = to_f64(q, dtype)
    out = np.empty(qf.shape, dtype=np.float64)
    for g in range(num_kv_heads):
        kf = to_f64(k[:, g, :], kv_dtype or dtype)
        vf = to_f64(v[:, g, :], kv_dtype or dtype)
        for i in range(q_len):
            last = L - q_len + i                      # row i sees 0..last
            rows = qf[i, g * G:(g + 1) * G, :]        # the G query heads of KV head g
            out[i, g * G:(g + 1) * G, :] = attend(rows, kf[:last + 1], vf[:last + 1], scale)
    return out


def _q_dtype(pool: HostPool, q_dtype):
    return q_dtype or ("bf16" if pool.dtype == "fp8" else pool.dtype)


def attention_paged_seq(q, pool: HostPool, table, ctx_len: int, q_len: int,
                        num_q_heads: int, scale: float, q_dtype: str = None) -> np.ndarray:
    """One sequence read through its block table: gather, then the definition.
    An fp8 pool is read as its dequantised values (code value times the
    token's scale)."""
    G = num_q_heads // pool.hkv
    qf = to_f64(q, _q_dtype(pool, q_dtype))
    out = np.empty(qf.shape, dtype=np.float64)
    for g in range(pool.hkv):
        kf, vf = pool.gather_head_f64(table, ctx_len, g)
        for i in range(q_len):
            last = ctx_len - q_len + i
            rows = qf[i, g * G:(g + 1) * G, :]
            out[i, g * G:(g + 1) * G, :] = attend(rows, kf[:last + 1], vf[:last + 1], scale)
    return out


def attention_paged(q, pool: HostPool, tables, ctx_lens, q_len: int, scale: float,
                    q_dtype: str = None) -> np.ndarray:
    """Batch form. q: [B][q_len][H_q][d]; tables: [B][MB] (int, -1 padded);
    ctx_lens: [B]. Returns float64 [B][q_len][H_q][d]."""
    B, _, Hq, _ = q.shape
    return np.stack([attention_paged_seq(q[b], pool, tables[b], int(ctx_lens[b]), q_len, Hq, scale, q_dtype)
                     for b in range(B)])
