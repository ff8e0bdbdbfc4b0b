"""Paged KV cache and paged decode attention for AMD Instinct MI355X (gfx950).

The compute runs in ``libpagedattn.so`` (HIP, built in-tree); this package is
its Python binding. Importing it loads the library or raises ImportError.
"""
from ._lib import (PA_DTYPE_BF16, PA_DTYPE_F32, PA_PATH_AUTO, PA_PATH_MFMA,  # noqa: F401
                   PA_SCHED_BALANCED, PA_SCHED_PARTITIONS, PA_SCHED_PARTITIONS_WAVE, PA_DTYPE_FP8_E4M3, PA_KV_SAME,
                   PA_KV_FP8_E4M3, PA_TREE_MAX_NODES,
                   PA_PATH_VALU, AttnDesc, AttnPlan, LIB_PATH)
from .api import *  # noqa: F401,F403
from .cache import PagedKVCache  # noqa: F401
