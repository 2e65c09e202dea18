"""Base model lm_head over the tree nodes -- TEST INFRASTRUCTURE ONLY.

The pages' verify step runs the base model over every tree node
([API] tree_decoding returns the base model's logits at each node) and hands
those logits to the acceptance test ([API] evaluate_posterior).  The base
lm_head is a plain linear map without bias (LLaMA's output projection, the
model the pages' Medusa heads sit on): logits[m][v] = sum_k hidden[m][k] *
W[v][k], W stored out x in.

fp64 from the exact input values (bf16 bits or float32 values).
"""

import numpy as np

from .common import as_f64
from .posterior import evaluate_posterior


def base_logits(hidden, w_base):
    """hidden [M][H], w_base [V][H] -> logits [M][V], float64."""
    h = as_f64(hidden)
    w = as_f64(w_base)
    return h @ w.T


def base_posterior(hidden, w_base, tree_candidates, retrieve, num_paths, temperature, eps, delta):
    """The acceptance test on the base logits of every tree node.

    hidden [B][T][H] (node order), w_base [V][H].  The logits are rounded to
    float32 first, as a caller that materialises them would hand them over.
    """
    B, T, H = np.asarray(hidden).shape
    z = base_logits(np.asarray(hidden).reshape(B * T, H), w_base).reshape(B, T, -1)
    return evaluate_posterior(z.astype(np.float32), tree_candidates, retrieve, num_paths, temperature, eps, delta)
