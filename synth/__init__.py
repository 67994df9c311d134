"""Seeded synthetic inputs for the routed-expert MoE layer.

This package only draws inputs: weights (packed into layer-expert records),
router matrices, hidden states and, where routing is bypassed, routes.  It
contains none of the layer's arithmetic, and both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from here.

Randomness is a counter-based SplitMix64 stream per (config, tensor, layer,
expert) key, implemented in ``gen.c``; distributions come from 65536-entry
inverse-CDF tables, so every byte is a pure function of its key and index.
"""
from .configs import CONFIGS, MoEConfig, record_bytes  # noqa: F401
from .inputs import (  # noqa: F401
    bank, record, router, tokens, ar1_tokens, zipf_routes, f32_to_bf16, bf16_to_f32,
    normal_table_bf16, normal_table_f32, e8m0_table, FMT_CODES, logical_streams,
)
