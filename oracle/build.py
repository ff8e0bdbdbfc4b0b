"""Fill the host pool model for a workload, in the workloads' fixed order.

Order (the pages give none; this fixed order makes every allocation unique):
  * without a shared prefix: sequences b = 0..B-1 each write their whole
    context starting at position 0;
  * with a shared prefix (Blog #54, interview question 2: requests that share
    a prompt point at the same physical blocks; Part 8, "RadixAttention": a
    reuse increments ref_count): sequence 0 writes the prefix, every other
    sequence forks each prefix block into its own table, then sequences
    b = 0..B-1 write their private tokens after the prefix (a private write
    into a shared, partly filled last prefix block copies it first).
``shared_prefix=False`` writes a private copy of the prefix per sequence
instead; the attention result must not change.
"""
from __future__ import annotations

import numpy as np

from workloads import Workload

from .allocator import BlockPoolModel
from .store import HostPool


def build_pool(w: Workload, shared_prefix: bool = True, fill_nan: bool = True):
    cfg = w.cfg
    B, MB = cfg.batch, w.max_blocks
    model = BlockPoolModel(w.num_blocks, cfg.block_size, w.free_order)
    pool = HostPool(w.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.kv_dtype or cfg.dtype,
                    fill_nan)
    tables = [[-1] * MB for _ in range(B)]
    live = [0] * B
    if cfg.prefix_len and shared_prefix:
        live[0] = pool.write(model, tables[0], MB, 0, 0, w.prefix_k, w.prefix_v)
        for b in range(1, B):
            for j in range(live[0]):
                model.fork(tables[0][j])
                tables[b][j] = tables[0][j]
            live[b] = live[0]
    elif cfg.prefix_len:
        for b in range(B):
            live[b] = pool.write(model, tables[b], MB, 0, 0, w.prefix_k, w.prefix_v)
    for b in range(B):
        s = w.seqs[b]
        live[b] = pool.write(model, tables[b], MB, live[b], cfg.prefix_len, s.k, s.v)
    return pool, model, np.asarray(tables, dtype=np.int32), live
