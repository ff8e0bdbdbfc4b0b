"""ctypes loader for libpagedattn.so (built in-tree by ``build.py``).

Importing this module loads the HIP library or raises: there is no CPU
fallback for any call.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

(PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_NO_FREE_BLOCK, PA_ERR_BAD_BLOCK, PA_ERR_HIP, PA_ERR_NO_MEMORY,
 PA_ERR_TOO_LARGE) = range(8)
PA_NOALLOC_SCRATCH_BYTES = 64 << 20
PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3 = 0, 1, 2
PA_KV_SAME, PA_KV_FP8_E4M3 = 0, 1
PA_PATH_AUTO, PA_PATH_VALU, PA_PATH_MFMA = 0, 1, 2
PA_SCHED_PARTITIONS, PA_SCHED_BALANCED, PA_SCHED_PARTITIONS_WAVE = 0, 1, 2
PA_TREE_MAX_NODES = 32

i32, i64, vp, f32, sz = C.c_int32, C.c_int64, C.c_void_p, C.c_float, C.c_size_t
pi32 = C.POINTER(C.c_int32)


class AttnDesc(C.Structure):
    _fields_ = [("num_seqs", i32), ("num_q_heads", i32), ("num_kv_heads", i32),
                ("head_dim", i32), ("block_size", i32), ("max_blocks_per_seq", i32),
                ("num_blocks", i32), ("dtype", i32), ("max_context", i32), ("path", i32),
                ("partition_tokens", i32), ("waves_per_group", i32), ("kv_shared", i32),
                ("kv_format", i32), ("reserved", i32 * 2)]


class AttnPlan(C.Structure):
    _fields_ = [("path", i32), ("schedule", i32), ("partition_tokens", i32), ("num_partitions", i32),
                ("waves_per_group", i32), ("grid", i32), ("merge_grid", i32),
                ("tiles_per_wave", i32), ("partitions_per_wave", i32), ("segment_cost", i32),
                ("workspace_bytes", sz)]


# (name, restype, argtypes) of every exported entry point
SIGNATURES = [
    ("pa_status_string", C.c_char_p, [i32]),
    ("pa_pool_create", i32, [i32, i32, i32, i32, i32, pi32, C.POINTER(vp)]),
    ("pa_pool_destroy", None, [vp]),
    ("pa_kv_bytes_per_token", i64, [i32, i32, i32, i32]),
    ("pa_pool_buffer_bytes", i64, [i32, i32, i32, i32, i32]),
    ("pa_block_alloc", i32, [vp, pi32]),
    ("pa_block_fork", i32, [vp, i32]),
    ("pa_block_free", i32, [vp, i32]),
    ("pa_block_refcount", i32, [vp, i32, pi32]),
    ("pa_pool_num_free", i32, [vp, pi32]),
    ("pa_pool_free_list", i32, [vp, pi32, i32, pi32]),
    ("pa_write_plan", i32, [vp, pi32, i32, pi32, i32, i32, pi32, i32, pi32, pi32]),
    ("pa_write_kv", i32, [vp, vp, vp, pi32, i32, pi32, i32, i32, vp, vp, vp]),
    ("pa_copy_blocks", i32, [vp, vp, vp, pi32, i32, vp]),
    ("pa_attention_plan", i32, [C.POINTER(AttnDesc), i32, C.POINTER(AttnPlan)]),
    ("pa_attention_workspace_size", sz, [C.POINTER(AttnDesc), i32]),
    ("pa_attention", i32, [C.POINTER(AttnDesc), vp, vp, vp, vp, vp, i32, f32, vp, vp, sz, vp]),
    ("pa_attention_noalloc", i32, [C.POINTER(AttnDesc), vp, vp, vp, vp, vp, i32, f32, vp, vp]),
    ("pa_attention_tree", i32, [C.POINTER(AttnDesc), vp, vp, vp, vp, vp, i32, vp, i32, f32, vp, vp, sz, vp]),
    ("pa_tree_masks", i32, [pi32, i32, C.POINTER(C.c_uint32)]),
    ("pa_spec_accept", i32, [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]),
    ("pa_spec_accept_workspace_size", sz, [i32, i32]),
    ("pa_prefix_cache_create", i32, [vp, C.POINTER(vp)]),
    ("pa_prefix_cache_destroy", None, [vp]),
    ("pa_prefix_match", i32, [vp, pi32, i32, pi32, i32, pi32]),
    ("pa_prefix_insert", i32, [vp, pi32, i32, pi32, i32, pi32]),
    ("pa_prefix_evict", i32, [vp, i32, pi32, pi32]),
    ("pa_prefix_cache_stats", i32, [vp, pi32, pi32, pi32]),
    ("pa_prefix_cache_dump", i32, [vp, pi32, pi32, C.POINTER(i64), i32, pi32]),
    ("pa_read_probe", i32, [vp, i64, i32, vp, i32, i32, vp, vp]),
    ("pa_last_hip_error", i32, []),
    ("pa_hip_error_name", C.c_char_p, [i32]),
]


def _load() -> C.CDLL:
    # torch ships its own HIP runtime under the same soname as ROCm's. Loading
    # torch first makes this library bind to that one runtime; loaded the other
    # way round the process holds two HIP runtimes, and device pointers and
    # streams from torch mean nothing to the library's (hipErrorNoDevice).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_218_amd.build` "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = C.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
