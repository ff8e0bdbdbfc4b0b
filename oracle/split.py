"""Split-KV attention: partition-local results and their log-sum-exp merge.

Page "Mở rộng Quy mô và Triển khai", section "Song song hóa Chuỗi (Sequence
Parallelism)": the cached keys/values of one long sequence are split into
segments, attention is computed locally on each segment and a reduction then
combines the local results. The pages do not write the reduction out (they
name the online softmax in Part 8, "Thực Thi Kernel Toán Học Trong CUDA", but
do not print it). The reading here is the standard exact one: a segment p
reports its score maximum m_p, its sum of exponentials l_p = sum exp(s - m_p)
and its normalised output o_p = sum exp(s - m_p) v / l_p; the merge rescales
each segment to the global maximum M:
    w_p = l_p * exp(m_p - M),   out = sum_p w_p o_p / sum_p w_p.
Empty segments contribute nothing.
"""
from __future__ import annotations

import numpy as np


def partition_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       part_tokens: int):
    """q [R][d], k/v [T][d] (float64). Returns m [P][R], l [P][R], o [P][R][d]."""
    T = k.shape[0]
    P = -(-T // part_tokens)
    R, d = q.shape
    m = np.empty((P, R))
    l = np.empty((P, R))
    o = np.empty((P, R, d))
    for p in range(P):
        ks = k[p * part_tokens:(p + 1) * part_tokens]
        vs = v[p * part_tokens:(p + 1) * part_tokens]
        s = scale * (q @ ks.T)
        m[p] = s.max(axis=-1)
        e = np.exp(s - m[p][:, None])
        l[p] = e.sum(axis=-1)
        o[p] = (e @ vs) / l[p][:, None]
    return m, l, o


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine P partition results: m, l [P][R], o [P][R][d] -> [R][d]."""
    M = m.max(axis=0)
    w = l * np.exp(m - M[None, :])
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]


def attend_split(q, k, v, scale: float, part_tokens: int) -> np.ndarray:
    return lse_merge(*partition_partials(q, k, v, scale, part_tokens))
