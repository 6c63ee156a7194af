"""Seeded synthetic inputs for verification attention over a paged KV cache.

This module only draws and lays out inputs (page pools, page tables, lengths,
draft trees, packed masks, quantised caches, new draft keys/values, RoPE cos/sin rows of token positions). It holds none of the attention
arithmetic, so both the CPU oracle and the GPU path can consume what it makes
without sharing any of the method's code.
"""

from .gen import (  # noqa: F401
    Problem,
    CONFIG_NAMES,
    make_case,
    make_config,
    random_tree_parents,
    tree_mask_rows,
    chain_parents,
    pack_mask_rows,
    poison_unused,
    problem_sha256,
    kv_bytes,
    make_append_inputs,
    rope_positions,
    rope_cos_sin,
    tree_depths,
)
