"""Pins for the oracle's Medusa heads.

Closed forms with single-entry weights fix the residual, the SiLU form and
the out x in orientation of W1 and the lm_head; a zero ResBlock reduces the
head to a textbook GEMV checked against an exactly rounded ``math.fsum``
dot product; top-k is checked against Python's ``sorted``.
"""

import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_zero_resblock_is_identity_and_plain_gemv():
    B, H, V, K = 2, 16, 12, 3
    h = _rand((B, H), 1)
    wlm = _rand((K, V, H), 2, 0.3)
    r = oracle.resblock(h, np.zeros((K, H, H)), np.zeros((K, H)))
    for j in range(K):
        assert np.array_equal(r[:, j, :], h)
    z = oracle.lm_head_logits(r, wlm)
    for b in range(B):
        for j in range(K):
            for v in range(V):
                want = math.fsum(float(wlm[j, v, c]) * float(h[b, c]) for c in range(H))
                assert abs(z[b, j, v] - want) <= 1e-13 * (1 + abs(want))


def test_silu_residual_and_w1_orientation():
    # W1[j] has one entry, at output row a and input column c, equal to ln 3.
    # With h[c] = 1: u[a] = ln 3, sigmoid(ln 3) = 3/4, so r[a] = h[a] + (3/4) ln 3;
    # every other row has u = 0 and r = h.
    H, a, c = 8, 5, 2
    h = _rand((1, H), 3)
    h[0, c] = 1.0
    w1 = np.zeros((2, H, H))
    w1[1, a, c] = math.log(3.0)
    r = oracle.resblock(h, w1, np.zeros((2, H)))
    expect = h[0].copy()
    expect[a] += 0.75 * math.log(3.0)
    assert np.allclose(r[0, 1], expect, rtol=0, atol=1e-15)
    assert np.array_equal(r[0, 0], h[0])


def test_silu_negative_branch_via_bias():
    # u = b1 = -ln 3: sigmoid(-ln 3) = 1/4, so SiLU(u) = -(ln 3)/4.
    H = 4
    h = _rand((1, H), 4)
    b1 = np.full((1, H), -math.log(3.0))
    r = oracle.resblock(h, np.zeros((1, H, H)), b1)
    assert np.allclose(r[0, 0], h[0] - math.log(3.0) / 4.0, rtol=0, atol=1e-15)


def test_silu_large_argument_limits():
    # SiLU(u) -> u for large u and -> 0 for very negative u.
    h = np.zeros((1, 2))
    b1 = np.array([[60.0, -60.0]])
    r = oracle.resblock(h, np.zeros((1, 2, 2)), b1)
    assert abs(r[0, 0, 0] - 60.0) < 1e-12
    assert abs(r[0, 0, 1]) < 1e-20


def test_lm_head_orientation():
    # Wlm[j] has one entry at vocab row v, hidden column c: z[v] = w * r[c], all else 0.
    B, H, V, K = 1, 6, 9, 2
    r = _rand((B, K, H), 5)
    wlm = np.zeros((K, V, H))
    wlm[1, 7, 4] = 2.5
    z = oracle.lm_head_logits(r, wlm)
    assert z[0, 1, 7] == 2.5 * r[0, 1, 4]
    z[0, 1, 7] = 0.0
    assert not np.any(z)


def test_topk_matches_sorted():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((3, 50))
    ids, vals = oracle.topk_by_value(z, 7)
    for row in range(3):
        want = sorted(range(50), key=lambda v: (-float(np.float32(z[row, v])), v))[:7]
        assert ids[row].tolist() == want
        assert np.array_equal(vals[row], z[row, want])


def test_topk_ties_lower_id_first():
    z = np.array([[1.0, 3.0, 2.0, 3.0, 3.0, 0.5]])
    ids, _ = oracle.topk_by_value(z, 4)
    assert ids[0].tolist() == [1, 3, 4, 2]


def test_topk_decides_in_float32():
    # 1 + 2^-30 and 1 differ in float64 but round to the same float32,
    # so the tie goes to the lower id.
    z = np.array([[1.0, 1.0 + 2.0 ** -30, 0.0]])
    ids, _ = oracle.topk_by_value(z, 2)
    assert ids[0].tolist() == [0, 1]


def test_heads_bf16_bits_decode():
    # bf16 bits 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25
    h = np.array([[0x3F80, 0xC000]], dtype=np.uint16)
    w1 = np.zeros((1, 2, 2), dtype=np.uint16)
    b1 = np.zeros((1, 2), dtype=np.uint16)
    wlm = np.array([[[0x3E80, 0x0000], [0x0000, 0x3F80]]], dtype=np.uint16)
    out = oracle.heads(h, w1, b1, wlm, topk=2, keep_logits=True)
    assert out["logits"][0, 0].tolist() == [0.25, -2.0]
    assert out["topk_ids"][0, 0].tolist() == [0, 1]


@pytest.mark.parametrize("j", [0, 2])
def test_heads_are_independent(j):
    B, H, V, K = 1, 8, 10, 3
    h = _rand((B, H), 7)
    w1 = _rand((K, H, H), 8, 0.1)
    b1 = _rand((K, H), 9, 0.1)
    wlm = _rand((K, V, H), 10, 0.3)
    base = oracle.heads(h, w1, b1, wlm, topk=3, keep_logits=True)
    w1b, wlmb = w1.copy(), wlm.copy()
    other = (j + 1) % K
    w1b[other] += 1.0
    wlmb[other] *= -1.0
    mod = oracle.heads(h, w1b, b1, wlmb, topk=3, keep_logits=True)
    assert np.array_equal(base["logits"][:, j], mod["logits"][:, j])
    assert not np.array_equal(base["logits"][:, other], mod["logits"][:, other])
