"""Python names for the C ABI (argument marshalling only).

Each function forwards to the ``pa_*`` entry point of the same name; device
buffers are torch tensors (their ``data_ptr()`` is passed), host arrays are
numpy int32 arrays, and the stream defaults to torch's current HIP stream.
A non-OK status raises ``PAError``.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np

from . import _lib
from ._lib import AttnDesc, AttnPlan, lib


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.pa_status_string(status).decode()
        if status == _lib.PA_ERR_HIP:
            e = lib.pa_last_hip_error()
            msg += f" [{lib.pa_hip_error_name(e).decode()} ({e})]"
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.PA_OK:
        raise PAError(status, where)


def _i32p(arr: Optional[np.ndarray]):
    if arr is None:
        return None
    assert arr.dtype == np.int32 and arr.flags.c_contiguous
    return arr.ctypes.data_as(_lib.pi32)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.float32:
        return _lib.PA_DTYPE_F32
    if torch_dtype == torch.bfloat16:
        return _lib.PA_DTYPE_BF16
    raise ValueError(f"unsupported dtype {torch_dtype}")


# -- pool -------------------------------------------------------------------

class Pool:
    """Owned pa_pool handle (host metadata only)."""

    def __init__(self, handle: int):
        self.handle = handle

    # bound at import: a handle that lives until interpreter exit is released
    # after the module's globals are gone
    _destroy = staticmethod(lib.pa_pool_destroy)

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


class PrefixCache:
    """Owned pa_prefix_cache handle; keeps its pool alive."""

    def __init__(self, handle: int, pool: "Pool"):
        self.handle = handle
        self.pool = pool

    _destroy = staticmethod(lib.pa_prefix_cache_destroy)  # bound at import, as for Pool

    def __del__(self):
        if getattr(self, "handle", None) and getattr(getattr(self, "pool", None), "handle", None):
            self._destroy(self.handle)
            self.handle = None


def pa_status_string(status: int) -> str:
    return lib.pa_status_string(status).decode()


def pa_pool_create(num_blocks, block_size, num_kv_heads, head_dim, dtype, initial_free_order=None) -> Pool:
    out = C.c_void_p()
    order = None if initial_free_order is None else np.ascontiguousarray(initial_free_order, dtype=np.int32)
    _check(lib.pa_pool_create(num_blocks, block_size, num_kv_heads, head_dim, dtype, _i32p(order),
                              C.byref(out)), "pa_pool_create")
    return Pool(out.value)


def pa_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes) -> int:
    return lib.pa_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)


def pa_pool_buffer_bytes(num_blocks, block_size, num_kv_heads, head_dim, dtype) -> int:
    return lib.pa_pool_buffer_bytes(num_blocks, block_size, num_kv_heads, head_dim, dtype)


def pa_block_alloc(pool: Pool) -> int:
    b = C.c_int32()
    _check(lib.pa_block_alloc(pool.handle, C.byref(b)), "pa_block_alloc")
    return b.value


def pa_block_fork(pool: Pool, block_id: int) -> None:
    _check(lib.pa_block_fork(pool.handle, block_id), "pa_block_fork")


def pa_block_free(pool: Pool, block_id: int) -> None:
    _check(lib.pa_block_free(pool.handle, block_id), "pa_block_free")


def pa_block_refcount(pool: Pool, block_id: int) -> int:
    rc = C.c_int32()
    _check(lib.pa_block_refcount(pool.handle, block_id, C.byref(rc)), "pa_block_refcount")
    return rc.value


def pa_pool_num_free(pool: Pool) -> int:
    n = C.c_int32()
    _check(lib.pa_pool_num_free(pool.handle, C.byref(n)), "pa_pool_num_free")
    return n.value


def pa_pool_free_list(pool: Pool) -> np.ndarray:
    n = C.c_int32()
    cap = pa_pool_num_free(pool)
    out = np.zeros(max(cap, 1), dtype=np.int32)
    _check(lib.pa_pool_free_list(pool.handle, _i32p(out), cap, C.byref(n)), "pa_pool_free_list")
    return out[:n.value].copy()


def pa_write_plan(pool: Pool, block_table: np.ndarray, num_blocks: int, start_pos: int, n_tokens: int,
                  max_copies: int = 1024):
    """Returns (new live-block count, copies [(src, dst)], slots[n_tokens]); patches block_table."""
    live = C.c_int32(num_blocks)
    copies = np.zeros(2 * max_copies, dtype=np.int32)
    ncp = C.c_int32()
    slots = np.zeros(max(n_tokens, 1), dtype=np.int32)
    _check(lib.pa_write_plan(pool.handle, _i32p(block_table), block_table.size, C.byref(live), start_pos,
                             n_tokens, _i32p(copies), max_copies, C.byref(ncp), _i32p(slots)),
           "pa_write_plan")
    pairs = [(int(copies[2 * k]), int(copies[2 * k + 1])) for k in range(ncp.value)]
    return live.value, pairs, slots[:n_tokens].copy()


def pa_write_kv(pool: Pool, k_pool, v_pool, block_table: np.ndarray, num_blocks: int, start_pos: int,
                k_new, v_new, stream=None) -> int:
    """Returns the new live-block count; patches block_table (host int32 row)."""
    live = C.c_int32(num_blocks)
    n = 0 if k_new is None else int(k_new.shape[0])
    _check(lib.pa_write_kv(pool.handle, _ptr(k_pool), _ptr(v_pool), _i32p(block_table), block_table.size,
                           C.byref(live), start_pos, n, _ptr(k_new), _ptr(v_new), _stream(stream)),
           "pa_write_kv")
    return live.value


def pa_copy_blocks(pool: Pool, k_pool, v_pool, src_dst: np.ndarray, stream=None) -> None:
    arr = np.ascontiguousarray(src_dst, dtype=np.int32).reshape(-1)
    _check(lib.pa_copy_blocks(pool.handle, _ptr(k_pool), _ptr(v_pool), _i32p(arr), arr.size // 2,
                              _stream(stream)), "pa_copy_blocks")


# -- attention ----------------------------------------------------------------

def make_desc(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
              dtype, max_context, path=_lib.PA_PATH_AUTO, partition_tokens=0, waves_per_group=0,
              kv_shared=0, kv_format=_lib.PA_KV_SAME) -> AttnDesc:
    d = AttnDesc()
    d.num_seqs, d.num_q_heads, d.num_kv_heads = num_seqs, num_q_heads, num_kv_heads
    d.head_dim, d.block_size, d.max_blocks_per_seq = head_dim, block_size, max_blocks_per_seq
    d.num_blocks, d.dtype, d.max_context = num_blocks, dtype, max_context
    d.path, d.partition_tokens, d.waves_per_group = path, partition_tokens, waves_per_group
    d.kv_shared, d.kv_format = kv_shared, kv_format
    return d


def pa_attention_plan(desc: AttnDesc, q_len: int) -> AttnPlan:
    plan = AttnPlan()
    _check(lib.pa_attention_plan(C.byref(desc), q_len, C.byref(plan)), "pa_attention_plan")
    return plan


def pa_attention_workspace_size(desc: AttnDesc, q_len: int) -> int:
    return int(lib.pa_attention_workspace_size(C.byref(desc), q_len))


def pa_attention(desc: AttnDesc, q, k_pool, v_pool, block_tables, context_lens, q_len: int, scale: float,
                 out, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_attention(C.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                            _ptr(context_lens), q_len, scale, _ptr(out), _ptr(workspace), ws_bytes,
                            _stream(stream)), "pa_attention")


def pa_attention_noalloc(desc: AttnDesc, q, k_pool, v_pool, block_tables, context_lens, q_len: int,
                         scale: float, out, stream=None) -> None:
    _check(lib.pa_attention_noalloc(C.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                    _ptr(context_lens), q_len, scale, _ptr(out), _stream(stream)),
           "pa_attention_noalloc")


def pa_attention_tree(desc: AttnDesc, q, k_pool, v_pool, block_tables, context_lens, q_len: int,
                      tree_mask, mask_stride: int, scale: float, out, workspace=None, stream=None) -> None:
    """tree_mask: device uint32 masks, [B][mask_stride] or [q_len] when mask_stride is 0
    (a torch int32/uint32 tensor; only its bits matter)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_attention_tree(C.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                 _ptr(context_lens), q_len, _ptr(tree_mask), mask_stride, scale, _ptr(out),
                                 _ptr(workspace), ws_bytes, _stream(stream)), "pa_attention_tree")


def pa_tree_masks(parents: np.ndarray) -> np.ndarray:
    """Ancestor masks (uint32 [n]) of a tree given by parent indices (int32 [n])."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    masks = np.zeros(parents.size, dtype=np.uint32)
    _check(lib.pa_tree_masks(_i32p(parents), parents.size, masks.ctypes.data_as(C.POINTER(C.c_uint32))),
           "pa_tree_masks")
    return masks


def pa_spec_accept_workspace_size(num_seqs: int, vocab: int) -> int:
    return int(lib.pa_spec_accept_workspace_size(num_seqs, vocab))


def pa_spec_accept(p, q, draft, u_accept, u_draw, num_accepted, tokens, workspace, stream=None) -> None:
    """Device tensors: p float32 [B][K+1][V], q float32 [B][K][V], draft int32 [B][K],
    u_accept float32 [B][K], u_draw int32/uint32 [B] (bits); outputs num_accepted
    int32 [B], tokens int32 [B][K+1]; workspace: zero-filled before first use, at
    least pa_spec_accept_workspace_size(B, V) bytes."""
    B, K1, V = p.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pa_spec_accept(_ptr(p), _ptr(q), _ptr(draft), _ptr(u_accept), _ptr(u_draw), B, K1 - 1, V,
                              _ptr(num_accepted), _ptr(tokens), _ptr(workspace), ws_bytes, _stream(stream)),
           "pa_spec_accept")


# -- measurement aid -----------------------------------------------------------

def pa_read_probe(buf, order, blocks_in_flight: int, workgroups: int, sink, stream=None,
                  block_bytes: int = 8192) -> None:
    """Read the device tensor `buf` (>= order.numel() * block_bytes bytes) as
    blocks of block_bytes (4096 or 8192) in the order of the int32 device
    tensor `order`; sink: int32/uint32 device tensor of one element."""
    _check(lib.pa_read_probe(_ptr(buf), int(order.numel()), int(block_bytes), _ptr(order), blocks_in_flight,
                             workgroups, _ptr(sink), _stream(stream)), "pa_read_probe")


# -- radix prefix cache -------------------------------------------------------

def pa_prefix_cache_create(pool: Pool) -> PrefixCache:
    h = C.c_void_p()
    _check(lib.pa_prefix_cache_create(pool.handle, C.byref(h)), "pa_prefix_cache_create")
    return PrefixCache(h.value, pool)


def pa_prefix_cache_destroy(cache: PrefixCache) -> None:
    if cache.handle:
        lib.pa_prefix_cache_destroy(cache.handle)
        cache.handle = None


def _tokens(tokens) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))


def pa_prefix_match(cache: PrefixCache, tokens, table: np.ndarray) -> int:
    """Fills table[0..n) with the longest cached prefix (at most table.size blocks); returns n."""
    t = _tokens(tokens)
    n = C.c_int32()
    _check(lib.pa_prefix_match(cache.handle, _i32p(t), t.size, _i32p(table), table.size, C.byref(n)),
           "pa_prefix_match")
    return n.value


def pa_prefix_insert(cache: PrefixCache, tokens, table: np.ndarray, num_blocks: int) -> int:
    t = _tokens(tokens)
    n = C.c_int32()
    _check(lib.pa_prefix_insert(cache.handle, _i32p(t), t.size, _i32p(table), num_blocks, C.byref(n)),
           "pa_prefix_insert")
    return n.value


def pa_prefix_evict(cache: PrefixCache, max_blocks: int) -> list:
    out = np.zeros(max(max_blocks, 1), dtype=np.int32)
    n = C.c_int32()
    _check(lib.pa_prefix_evict(cache.handle, max_blocks, _i32p(out), C.byref(n)), "pa_prefix_evict")
    return out[:n.value].tolist()


def pa_prefix_cache_stats(cache: PrefixCache):
    a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib.pa_prefix_cache_stats(cache.handle, C.byref(a), C.byref(b), C.byref(c)), "pa_prefix_cache_stats")
    return a.value, b.value, c.value


def pa_prefix_cache_dump(cache: PrefixCache) -> list:
    """[(block, parent or -1, unreferenced stamp or -1)] in ascending block order."""
    n = C.c_int32()
    lib.pa_prefix_cache_dump(cache.handle, None, None, None, 0, C.byref(n))
    k = n.value
    blocks, parents = np.zeros(max(k, 1), np.int32), np.zeros(max(k, 1), np.int32)
    stamps = np.zeros(max(k, 1), np.int64)
    _check(lib.pa_prefix_cache_dump(cache.handle, _i32p(blocks), _i32p(parents),
                                    stamps.ctypes.data_as(C.POINTER(C.c_int64)), k, C.byref(n)),
           "pa_prefix_cache_dump")
    return [(int(blocks[i]), int(parents[i]), int(stamps[i])) for i in range(k)]
