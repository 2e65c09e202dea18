"""Seeded synthetic inputs for the Medusa verify step.

This package is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It only *draws* inputs (normal variates, random tree shapes,
token ids, RoPE-rotated query/key rows, planted acceptance paths) and encodes
them as fp32 or bf16 bits.  It holds none of the verify step's arithmetic:
no head GEMV, no tree construction, no attention, no acceptance rule and no
KV gather.  Where an input depends on the tree's node order (RoPE positions,
a planted path), the caller passes that structure in.  For tree-shape sweeps
it also holds a synthetic acceptance model (how likely each head rank is to
be right), used to pick and score tree specifications.

Every stream is keyed by ``SeedSequence(seed, spawn_key=(workload, tensor,
...))`` so any tensor can be regenerated alone and the same bits reach both
sides of a parity test.
"""

from .rng import stream, normal_f32, bf16_bits, bf16_to_f32, f32_round
from .shapes import WORKLOADS, workload
from .trees import (full_tree_choices, random_tree_choices, worked_example_choices,
                    chain_choices, choices_array, geometric_acceptance, path_probability,
                    best_tree_choices, expected_accept_length)
from .gen import (base_head_inputs, base_posterior_inputs, heads_inputs, topk_ids_input, root_token_input, attention_inputs,
                  posterior_logits, kv_cache, rope_rotate, prefix_lengths, node_uniforms, tiny_decoder,
                  tiny_heads)

__all__ = [
    "stream", "normal_f32", "bf16_bits", "bf16_to_f32", "f32_round",
    "WORKLOADS", "workload",
    "full_tree_choices", "random_tree_choices", "worked_example_choices", "chain_choices",
    "choices_array", "geometric_acceptance", "path_probability", "best_tree_choices",
    "expected_accept_length",
    "base_head_inputs", "base_posterior_inputs", "heads_inputs", "topk_ids_input", "root_token_input", "attention_inputs",
    "posterior_logits", "kv_cache", "rope_rotate", "prefix_lengths", "node_uniforms", "tiny_decoder",
    "tiny_heads",
]
