"""Seeded synthetic workloads for the tree-verification step (inputs only).

This package is the single source of inputs shared by the CPU oracle, the
GPU parity tests and the benchmark.  It draws tensors, token trees and random
coins; it computes nothing that the verification method computes (no
attention, no logits, no acceptance, no cache moves).
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    attn_inputs,
    draft_coins,
    draft_tokens,
    lmhead_inputs,
    paged_layout,
    TREE_BUILDS,
    TreeBuildConfig,
    draft_logp,
    PathDrafter,
    bf16_bits_from_f32,
    BF16_QNAN,
)
from .model import MODEL_CASES, MODELS, ModelConfig, model_inputs, model_weights  # noqa: F401
