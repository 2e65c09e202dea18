"""CPU oracle for the Medusa verify step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 restatement of what each stage of the verify step
computes, written from the pages' descriptions of Medusa:

  heads.py      ResBlock heads, per-head lm_head logits and top-k
  tree.py       the candidate tree from a ``medusa_choices`` spec
  attention.py  tree-masked attention over a KV prefix
  posterior.py  greedy / typical acceptance and the longest accepted prefix
  nucleus.py    nucleus (top-p) acceptance: a sample per node, children
                accepted when they equal their parent's sample
  sampling.py   Philox4x64-10 uniforms keyed by (seed, step, sequence,
                node, purpose) and the typical-mode sampled next token
  commit.py     gathering the accepted path's K/V into contiguous slots
  base_head.py  the base model's lm_head over the tree nodes, and the
                acceptance test on its logits
  decoder.py    a tiny LLaMA-style base model (whole-sequence forward) and
                its plain greedy decoding

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the GPU library and imports neither it
nor the synthetic-input package; the two sides meet only on the same input
bits.

Precision: every computation is float64 from the exact input values (bf16
bits or float32 values).  Where a float result decides an integer (top-k
order, an acceptance test) the decision is taken on float32-rounded values,
the precision the GPU kernels decide in.

Every function here is pinned by tests that do not reuse its code (worked
example, closed forms, brute force on tiny inputs, library special cases);
no function is parity-unpinned.
"""

from .common import as_f64
from .heads import resblock, lm_head_logits, topk_by_value, heads
from .tree import SpecError, parse_choices, build_tree
from .attention import tree_attention
from .posterior import node_statistics, evaluate_posterior
from .commit import commit_kv
from .base_head import base_logits, base_posterior
from .nucleus import nucleus, nucleus_sample, evaluate_posterior_nucleus
from . import sampling
from . import decoder

__all__ = [
    "as_f64", "resblock", "lm_head_logits", "topk_by_value", "heads",
    "SpecError", "parse_choices", "build_tree", "tree_attention",
    "node_statistics", "evaluate_posterior", "commit_kv", "base_logits", "base_posterior",
    "nucleus", "nucleus_sample", "evaluate_posterior_nucleus", "sampling", "decoder",
]
