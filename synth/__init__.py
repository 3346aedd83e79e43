"""Seeded synthetic workloads for speculative verify and the P-EAGLE draft batch.

This package only draws inputs: target logits, draft distributions and draft
tokens, uniforms, hidden states, prompt lengths and block tables.  It holds
none of the verify or batch-construction arithmetic; both the HIP path and the
CPU oracle receive the arrays it returns.
"""
from .workloads import (  # noqa: F401
    BuildInputs,
    VerifyInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_build_inputs,
    make_verify_inputs,
    make_fused_inputs,
    DraftInputs,
    DraftSpec,
    DRAFT_CONFIGS,
    make_draft_inputs,
    make_temperatures,
    TreeInputs,
    TreeSpec,
    TREE_CONFIGS,
    make_tree_inputs,
    static_tree_parents,
    MIXED_TEMPERATURES,
    verify_config,
    build_config,
    CONFIG_NAMES,
)
