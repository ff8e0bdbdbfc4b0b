"""Host model of the paged K/V pool: physical layout, writes and the gather.

Layout (the library's documented pool layout, so that device pools can be
compared with this model byte for byte):
    k[block][kv_head][dim // 32][slot_in_block][dim % 32]   ([NB][H_kv][d/32][bs][32])
    v[block][kv_head][dim][slot_in_block]                   ([NB][H_kv][d][bs])
(K's head dimension is cut into 32-element slabs; each slab keeps the block's
tokens one after another.)
FP8 pools ("fp8", OCP E4M3 codes with one fp32 scale per token and KV head):
    k[block][kv_head][dim // 64][slot_in_block][dim % 64]   uint8 codes
    v[block][kv_head][dim][slot_in_block]                   uint8 codes
    k_scale[block][kv_head][slot_in_block], v_scale[...]     fp32
Rows written to an fp8 pool arrive as bf16 bit patterns and are quantised
per (token, KV head) by oracle.fp8.quantize_rows.
Physical slot s = block * bs + offset holds token position p of a sequence
whose table maps logical block p // bs to ``block`` and offset = p % bs
(block table / free pool: Part 8, "Phân Tích Cơ Cấu Bộ Nhớ Của KV Cache"
diagram; Blog #54, section 2.2). Unwritten slots keep the fill value (NaN in
tests), which the attention result must never depend on.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .allocator import BlockPoolModel
from .numerics import to_f64

_NAN_BITS = {"bf16": np.uint16(0x7FC0)}


class HostPool:
    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int,
                 head_dim: int, dtype: str, fill_nan: bool = True):
        self.nb, self.bs, self.hkv, self.d, self.dtype = num_blocks, block_size, num_kv_heads, head_dim, dtype
        assert head_dim % 32 == 0
        if dtype == "fp8":
            assert head_dim % 64 == 0
            code_fill = np.uint8(0x7F) if fill_nan else 0          # E4M3 NaN
            self.k = np.full((num_blocks, num_kv_heads, head_dim // 64, block_size, 64), code_fill, np.uint8)
            self.v = np.full((num_blocks, num_kv_heads, head_dim, block_size), code_fill, np.uint8)
            sfill = np.float32(np.nan) if fill_nan else np.float32(0)
            self.k_scale = np.full((num_blocks, num_kv_heads, block_size), sfill, np.float32)
            self.v_scale = np.full((num_blocks, num_kv_heads, block_size), sfill, np.float32)
            return
        np_t = np.float32 if dtype == "f32" else np.uint16
        fill = (np.float32(np.nan) if dtype == "f32" else _NAN_BITS["bf16"]) if fill_nan else 0
        self.k = np.full((num_blocks, num_kv_heads, head_dim // 32, block_size, 32), fill, dtype=np_t)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=np_t)

    @property
    def slab(self) -> int:
        return 64 if self.dtype == "fp8" else 32

    def copy_block(self, src: int, dst: int) -> None:
        self.k[dst] = self.k[src]
        self.v[dst] = self.v[src]
        if self.dtype == "fp8":
            self.k_scale[dst] = self.k_scale[src]
            self.v_scale[dst] = self.v_scale[src]

    def scatter(self, slots, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Store token rows k_new/v_new ([n][H_kv][d]) at the given physical slots."""
        slots = np.asarray(slots, dtype=np.int64)
        blk, off = slots // self.bs, slots % self.bs
        # slots are distinct, so the fancy-index assignment has no collisions
        n = slots.size
        if self.dtype == "fp8":
            kc, ks = fp8.quantize_rows(to_f64(k_new, "bf16").astype(np.float32))
            vc, vs = fp8.quantize_rows(to_f64(v_new, "bf16").astype(np.float32))
            self.k_scale[blk, :, off] = ks
            self.v_scale[blk, :, off] = vs
            k_new, v_new = kc, vc
        self.k[blk, :, :, off, :] = np.asarray(k_new).reshape(n, self.hkv, self.d // self.slab, self.slab)
        self.v[blk, :, :, off] = v_new

    def put_token(self, blk: int, off: int, k_row=None, v_row=None) -> None:
        """Store one token's K and/or V rows ([H_kv][d]) in slot off of block blk."""
        if self.dtype == "fp8":
            if k_row is not None:
                k_row, self.k_scale[blk, :, off] = fp8.quantize_rows(to_f64(k_row, "bf16").astype(np.float32))
            if v_row is not None:
                v_row, self.v_scale[blk, :, off] = fp8.quantize_rows(to_f64(v_row, "bf16").astype(np.float32))
        if k_row is not None:
            self.k[blk, :, :, off, :] = np.asarray(k_row).reshape(self.hkv, self.d // self.slab, self.slab)
        if v_row is not None:
            self.v[blk, :, :, off] = v_row

    def write(self, model: BlockPoolModel, table, capacity: int, num_blocks: int,
              start_pos: int, k_new: np.ndarray, v_new: np.ndarray) -> int:
        """Append/overwrite tokens of one sequence: allocate and copy-on-write
        through the allocator model, then store the rows. Returns the new
        live-block count."""
        n_live, plan = model.plan_write(table, capacity, num_blocks, start_pos, k_new.shape[0])
        for src, dst in plan.copies:
            self.copy_block(src, dst)
        self.scatter(plan.slots, k_new, v_new)
        return n_live

    def gather(self, table, ctx_len: int):
        """Contiguous K, V ([L][H_kv][d]) of a sequence, read through its table."""
        pos = np.arange(ctx_len)
        blk = np.asarray(table, dtype=np.int64)[pos // self.bs]
        off = pos % self.bs
        k = self.k[blk, :, :, off, :].reshape(ctx_len, self.hkv, self.d)   # [L][H_kv][d] (storage values)
        v = self.v[blk, :, :, off]                                         # [L][H_kv][d]
        return k, v

    def gather_head(self, table, ctx_len: int, g: int):
        """K, V ([L][d]) of KV head g only (bounded memory for long contexts)."""
        pos = np.arange(ctx_len)
        blk = np.asarray(table, dtype=np.int64)[pos // self.bs]
        off = pos % self.bs
        return self.k[blk, g, :, off, :].reshape(ctx_len, self.d), self.v[blk, g, :, off]

    def gather_head_f64(self, table, ctx_len: int, g: int):
        """K, V ([L][d]) of KV head g as float64 values (dequantised for fp8)."""
        kr, vr = self.gather_head(table, ctx_len, g)
        if self.dtype != "fp8":
            return to_f64(kr, self.dtype), to_f64(vr, self.dtype)
        pos = np.arange(ctx_len)
        blk = np.asarray(table, dtype=np.int64)[pos // self.bs]
        off = pos % self.bs
        return (fp8.dequantize(kr, self.k_scale[blk, g, off]), fp8.dequantize(vr, self.v_scale[blk, g, off]))
