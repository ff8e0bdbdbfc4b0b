"""A batch of sequences over one paged KV pool, driven through the C ABI.

Holds the pool handle (host refcounts and free list), the device K/V pools
(torch tensors, pool layout k [NB][H_kv][d/32][bs][32], v [NB][H_kv][d][bs];
FP8 pools are byte buffers of E4M3 codes followed by fp32 scales), the
host block tables and each sequence's live-block count. Every operation is
one ``pa_*`` call; torch only provides the device memory and the stream.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import _lib
from . import api


def _to_device(arr: np.ndarray, torch_dtype, device):
    import torch
    if torch_dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device, non_blocking=False)


class PagedKVCache:
    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, torch_dtype,
                 num_seqs: int, max_blocks: int, initial_free_order=None, device="cuda",
                 fill_nan: bool = True, kv_fp8: bool = False):
        """torch_dtype: the dtype of queries, outputs and written K/V rows;
        kv_fp8: the pools store E4M3 codes plus scales (rows written as bf16)."""
        import torch
        self.nb, self.bs, self.hkv, self.d = num_blocks, block_size, num_kv_heads, head_dim
        self.torch_dtype, self.device = torch_dtype, device
        self.dtype = api.dtype_code(torch_dtype)
        self.kv_fp8 = kv_fp8
        pool_dtype = _lib.PA_DTYPE_FP8_E4M3 if kv_fp8 else self.dtype
        self.pool = api.pa_pool_create(num_blocks, block_size, num_kv_heads, head_dim, pool_dtype,
                                       initial_free_order)
        if kv_fp8:
            nbytes = api.pa_pool_buffer_bytes(num_blocks, block_size, num_kv_heads, head_dim, pool_dtype)
            codes = num_blocks * num_kv_heads * block_size * head_dim
            self.k_pool = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.v_pool = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            if fill_nan:   # the E4M3 NaN code, and NaN scales
                for t in (self.k_pool, self.v_pool):
                    t[:codes].fill_(0x7F)
                    t[codes:].view(torch.float32).fill_(float("nan"))
        else:
            fill = float("nan") if fill_nan else 0.0
            self.k_pool = torch.full((num_blocks, num_kv_heads, head_dim // 32, block_size, 32), fill,
                                     dtype=torch_dtype, device=device)
            self.v_pool = torch.full((num_blocks, num_kv_heads, head_dim, block_size), fill,
                                     dtype=torch_dtype, device=device)
        self.tables = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
        self.live = [0] * num_seqs
        self.shared = False   # some block is (or was) in more than one table

    # -- writes -----------------------------------------------------------
    def write(self, b: int, start_pos: int, k_new, v_new, stream=None) -> None:
        """Store K/V rows ([n][H_kv][d] device tensors) at positions start_pos.."""
        row = self.tables[b]          # contiguous view; the library patches it in place
        self.live[b] = api.pa_write_kv(self.pool, self.k_pool, self.v_pool, row, self.live[b],
                                       start_pos, k_new, v_new, stream)

    # -- radix prefix cache ------------------------------------------------
    def enable_prefix_cache(self):
        self.prefix = api.pa_prefix_cache_create(self.pool)
        return self.prefix

    def match_prefix(self, b: int, tokens) -> int:
        """Sequence b (empty) starts with the longest cached prefix of tokens;
        returns the number of tokens it covers (write from there on)."""
        assert self.live[b] == 0
        n = api.pa_prefix_match(self.prefix, tokens, self.tables[b])
        self.live[b] = n
        self.shared = self.shared or n > 0
        return n * self.bs

    def insert_prefix(self, b: int, tokens) -> int:
        """Cache sequence b's full blocks of tokens (their K/V already written)."""
        return api.pa_prefix_insert(self.prefix, tokens, self.tables[b], self.live[b])

    def share_blocks(self, src: int, dst: int, n_blocks: int) -> None:
        """Sequence dst starts with the first n_blocks blocks of src (forked)."""
        for j in range(n_blocks):
            api.pa_block_fork(self.pool, int(self.tables[src, j]))
            self.tables[dst, j] = self.tables[src, j]
        self.live[dst] = n_blocks
        self.shared = self.shared or n_blocks > 0

    def free_seq(self, b: int) -> None:
        for j in range(self.live[b]):
            api.pa_block_free(self.pool, int(self.tables[b, j]))
        self.tables[b, :] = -1
        self.live[b] = 0

    def tables_device(self):
        import torch
        return torch.from_numpy(self.tables).to(self.device)

    # -- attention --------------------------------------------------------
    def desc(self, num_q_heads: int, max_context: int, path=_lib.PA_PATH_AUTO, partition_tokens=0,
             waves_per_group=0):
        return api.make_desc(self.tables.shape[0], num_q_heads, self.hkv, self.d, self.bs,
                             self.tables.shape[1], self.nb, self.dtype, max_context, path, partition_tokens,
                             waves_per_group, int(self.shared),
                             _lib.PA_KV_FP8_E4M3 if self.kv_fp8 else _lib.PA_KV_SAME)

    def attention(self, q, tables_dev, lens_dev, q_len: int, scale: float, max_context: int,
                  path=_lib.PA_PATH_AUTO, partition_tokens=0, waves_per_group=0, out=None, workspace=None,
                  stream=None, tree_mask=None, mask_stride=None):
        """pa_attention, or pa_attention_tree when tree_mask (device uint32/int32
        masks, [B][q_len] by default) is given."""
        import torch
        desc = self.desc(q.shape[2], max_context, path, partition_tokens, waves_per_group)
        if out is None:
            out = torch.empty_like(q)
        need = api.pa_attention_workspace_size(desc, q_len)
        if workspace is None and need:
            workspace = self.workspace(need, q.device)
        if tree_mask is None:
            api.pa_attention(desc, q, self.k_pool, self.v_pool, tables_dev, lens_dev, q_len, scale, out,
                             workspace, stream)
        else:
            stride = q_len if mask_stride is None else mask_stride
            api.pa_attention_tree(desc, q, self.k_pool, self.v_pool, tables_dev, lens_dev, q_len, tree_mask,
                                  stride, scale, out, workspace, stream)
        return out

    def workspace(self, nbytes: int, device):
        """A zero-filled workspace of at least nbytes, kept for later calls (its
        arrival counters are left zero by every completed call)."""
        import torch
        ws = getattr(self, "_ws", None)
        if ws is None or ws.numel() < nbytes or ws.device != torch.device(device):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self._ws = ws
        return ws

    # -- a whole synthetic batch ---------------------------------------------
    @classmethod
    def from_workload(cls, w, device="cuda", shared_prefix: bool = True, fill_nan: bool = True):
        """Build the cache for a generated workload in its fixed order: with a
        shared prefix, sequence 0 writes it and the others fork its blocks;
        then each sequence writes its own tokens after the prefix."""
        import torch
        cfg = w.cfg
        tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        c = cls(w.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, tdt, cfg.batch,
                w.max_blocks, w.free_order, device, fill_nan, kv_fp8=cfg.kv_dtype == "fp8")
        if cfg.prefix_len:
            pk, pv = _to_device(w.prefix_k, tdt, device), _to_device(w.prefix_v, tdt, device)
            if shared_prefix:
                c.write(0, 0, pk, pv)
                nblk = math.ceil(cfg.prefix_len / cfg.block_size)
                for b in range(1, cfg.batch):
                    c.share_blocks(0, b, nblk)
            else:
                for b in range(cfg.batch):
                    c.write(b, 0, pk, pv)
        for b in range(cfg.batch):
            s = w.seqs[b]
            c.write(b, cfg.prefix_len, _to_device(s.k, tdt, device), _to_device(s.v, tdt, device))
        return c


def queries_to_device(w, device="cuda"):
    """[B][q_len][H_q][d] query tensor of a workload on the device."""
    import torch
    tdt = torch.float32 if w.cfg.dtype == "f32" else torch.bfloat16
    return _to_device(w.q_all(), tdt, device)


def lens_to_device(w, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(w.lens, dtype=np.int32)).to(device)


def tree_masks_to_device(parents, device="cuda"):
    """Parent indices [B][q_len] -> device int32 [B][q_len] ancestor masks
    (library helper pa_tree_masks, one tree per row)."""
    import torch
    parents = np.asarray(parents, dtype=np.int32)
    masks = np.stack([api.pa_tree_masks(p) for p in parents]).view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(masks)).to(device)
