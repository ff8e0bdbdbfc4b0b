"""Seeded synthetic inputs for paged decode attention.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, none of the allocator rules and none of the pool
layout. Both the fp64 oracle (``oracle/``) and the HIP path's tests and
bench take their inputs from here, so the two sides see the same bits.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    Workload,
    SeqData,
    bf16_bits_from_f32,
    config,
    context_lengths,
    free_order,
    generate,
    pool_blocks,
    sequence,
    tree_parents,
)
from .spec import SPEC_CONFIGS, SpecConfig, SpecInputs, generate_spec, spec_config  # noqa: F401,E402
