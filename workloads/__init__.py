"""Seeded synthetic inputs for the paged KV-cache decode path.

This package is the only code that both the CPU oracle checks and the GPU
path consume.  It draws random numbers and describes workload shapes and
operation scripts; it contains none of the method's arithmetic (no slot
mapping, no attention, no quantisation).
"""
from .configs import (  # noqa: F401
    PAGE_EXAMPLE_FREE_ORDER,
    WORKLOADS,
    Workload,
    beam_parents,
    cb_prefix_script,
    prefix_cache_prompts,
    workload,
)
from .generators import (  # noqa: F401
    FP8_E4M3_MAX,
    SEED_BASE,
    amax_scales,
    head_offsets,
    minmax_int8_params,
    free_order,
    normal_fp16,
    seed_for,
    uniform_ints,
)
