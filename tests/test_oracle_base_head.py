"""Pins for the oracle's base lm_head over the tree nodes.

Single-entry weights fix the out x in orientation (W[v][k] = 1 picks
hidden[:, k] into logit v); every logit of a random case matches an exactly
rounded ``math.fsum`` dot product to fp64 rounding; bf16 inputs decode to
their exact values; and the posterior on the base logits equals the
posterior on logits a caller would materialise in float32.
"""

import math

import numpy as np

import oracle


def test_single_entry_weights_pick_hidden_columns():
    M, H, V = 3, 8, 5
    h = np.arange(M * H, dtype=np.float64).reshape(M, H) - 7.0
    for v, k in [(0, 0), (4, 7), (2, 3)]:
        w = np.zeros((V, H))
        w[v, k] = 1.0
        z = oracle.base_logits(h, w)
        expect = np.zeros((M, V))
        expect[:, v] = h[:, k]
        assert np.array_equal(z, expect)


def test_logits_match_exactly_rounded_dot_products():
    rng = np.random.default_rng(3)
    M, H, V = 4, 37, 6
    h = rng.standard_normal((M, H))
    w = rng.standard_normal((V, H)) * 0.1
    z = oracle.base_logits(h, w)
    for m in range(M):
        for v in range(V):
            ref = math.fsum(float(h[m, k]) * float(w[v, k]) for k in range(H))
            assert abs(z[m, v] - ref) <= 1e-13 * max(1.0, abs(ref))


def test_bf16_inputs_decode_exactly():
    # bf16 0x3f80 = 1.0, 0xc000 = -2.0, 0x3e80 = 0.25
    h = np.array([[0x3F80, 0xC000]], dtype=np.uint16)
    w = np.array([[0x3E80, 0x3F80], [0x3F80, 0x3F80]], dtype=np.uint16)
    z = oracle.base_logits(h, w)
    assert np.array_equal(z, np.array([[1.0 * 0.25 - 2.0, 1.0 - 2.0]]))


def test_base_posterior_is_posterior_of_float32_logits():
    rng = np.random.default_rng(5)
    B, T, H, V = 1, 3, 16, 10
    h = rng.standard_normal((B, T, H))
    w = rng.standard_normal((V, H))
    cand = np.array([[7, 2, 5]], dtype=np.int32)
    retrieve = np.array([[0, 1, -1], [0, 2, -1]], dtype=np.int32)
    z = np.einsum("btk,vk->btv", h, w).astype(np.float32)
    for temp in (0.0, 0.7):
        got = oracle.base_posterior(h, w, cand, retrieve, 2, temp, 0.09, 0.3)
        ref = oracle.evaluate_posterior(z, cand, retrieve, 2, temp, 0.09, 0.3)
        for key in ("best_path", "accept_len", "next_token"):
            assert np.array_equal(got[key], ref[key])
