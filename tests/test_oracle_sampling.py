"""Pins for the oracle's counter-based uniforms and typical-mode sampling.

Each check stands outside the oracle's own code:
  * Philox4x64-10 against NumPy's Philox bit generator (Philox4x64-10 in
    NumPy; it advances its 256-bit counter before each block, so block c
    is the first block after counter c - 1), over zero, small, large and
    carrying counters and several keys, and against the zero-input answer
    the Random123 distribution publishes;
  * the uniforms: the top 24 bits of NumPy's first word, exact multiples of
    2^-24 in [0, 1), and different for different (step, sequence, node,
    purpose);
  * typical sampling in closed form: a dominant token is drawn whatever u;
    a flat row over V tokens admits every token (1/V > delta/V) and u picks
    token floor(u V); sixteen equal tokens and a 17th far below admit the
    sixteen (the entropy branch binds) and u picks among them in id order;
    a two-point (0.05, 0.95) row excludes 0.05 (the eps branch binds);
  * the allowed set equals the set of children the (separately pinned)
    typical acceptance accepts on a star tree whose children are all V
    tokens, on random rows;
  * inverse-CDF frequencies over a fine grid of u match p renormalised over
    the allowed set within one grid step;
  * the sampled next token is drawn at the last accepted node of the best
    path, with the purpose-1 uniform of node 0.
"""

import numpy as np
import pytest

import oracle
from oracle import sampling as smp

_MASK = (1 << 64) - 1


def _numpy_block(counter, key):
    """NumPy's Philox4x64-10 block at `counter` (its counter set one below)."""
    c = sum(int(x) << (64 * i) for i, x in enumerate(counter))
    c = (c - 1) & ((1 << 256) - 1)
    prev = np.array([(c >> (64 * i)) & _MASK for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array([int(k) for k in key], dtype=np.uint64), counter=prev)
    return [int(x) for x in g.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ([0, 0, 0, 0], [0, 0]),
    ([1, 0, 0, 0], [0x123456789abcdef0, 0x0fedcba987654321]),
    ([5, 3, 2, 1], [42, 0]),
    ([_MASK, _MASK, _MASK, _MASK], [_MASK, _MASK]),
    ([0, 1, 0, 0], [7, 11]),              # block after a carry out of word 0
    ([255, 15, 1000, 1], [2 ** 63 + 5, 0]),
])
def test_philox_matches_numpy(counter, key):
    assert smp.philox4x64(counter, key) == _numpy_block(counter, key)


def test_philox_published_zero_answer():
    assert smp.philox4x64([0, 0, 0, 0], [0, 0]) == [0x16554d9eca36314c, 0xdb20fe9d672d0fdc,
                                                   0xd7e772cee186176b, 0x7e68b68aec7ba23b]


def test_uniforms_are_numpys_top_24_bits():
    seed, step = 0xdeadbeef, 17
    for b, n, purpose in [(0, 0, 0), (3, 63, 0), (15, 255, 1), (1, 2, 1)]:
        w = _numpy_block([n, b, step, purpose], [seed, 0])[0]
        u = smp.uniform(seed, step, b, n, purpose)
        assert u.dtype == np.float32 and 0.0 <= u < 1.0
        assert int(u * 2 ** 24) == w >> 40 and float(u) * 2 ** 24 == int(u * 2 ** 24)
    U = smp.uniforms(9, 4, 3, 50, 0)
    assert U.shape == (3, 50) and len(np.unique(U)) == U.size
    assert not np.array_equal(U, smp.uniforms(9, 5, 3, 50, 0))
    assert not np.array_equal(U, smp.uniforms(9, 4, 3, 50, 1))
    assert abs(float(smp.uniforms(1, 0, 4, 256, 0).mean()) - 0.5) < 0.03


def test_typical_sample_closed_forms():
    V = 40
    row = np.zeros(V, dtype=np.float32)
    row[7] = 60.0
    for u in (0.0, 0.3, 0.999):
        assert smp.typical_sample(row, 1.0, 0.09, 0.3, u) == 7
    flat = np.zeros(V, dtype=np.float32)
    ids, _ = smp.typical_allowed(flat, 0.7, 0.09, 0.3)
    assert ids.tolist() == list(range(V))
    for k in range(V):
        assert smp.typical_sample(flat, 0.7, 0.09, 0.3, (k + 0.5) / V) == k
    sixteen = np.full(V, -300.0, dtype=np.float32)
    members = [1, 3, 4, 8, 9, 10, 12, 15, 17, 20, 22, 25, 30, 33, 36, 39]
    sixteen[members] = 2.0
    ids, p = smp.typical_allowed(sixteen, 1.0, 0.09, 0.3)
    assert ids.tolist() == members and np.allclose(p, 1 / 16)
    for k in range(16):
        assert smp.typical_sample(sixteen, 1.0, 0.09, 0.3, (k + 0.25) / 16) == members[k]
    two = np.full(V, -500.0, dtype=np.float32)
    two[0], two[1] = np.log(0.05), np.log(0.95)
    ids, _ = smp.typical_allowed(two, 1.0, 0.09, 0.3)
    assert ids.tolist() == [1]
    assert smp.typical_sample(two, 1.0, 0.09, 0.3, 0.01) == 1


@pytest.mark.parametrize("seed", range(4))
def test_allowed_set_is_what_typical_acceptance_accepts(seed):
    rng = np.random.default_rng(seed)
    V = 300
    row = (rng.standard_normal(V) * (1.5 + seed)).astype(np.float32)
    t = 0.7
    ids, _ = smp.typical_allowed(row, t, 0.09, 0.3)
    # a star tree with every token as a child of the root: the accepted
    # children are exactly the allowed tokens
    T = 1 + V
    cand = np.array([[0] + list(range(V))], dtype=np.int32)
    retrieve = np.array([[0, 1 + v] for v in range(V)], dtype=np.int32)
    logits = np.zeros((1, T, V), dtype=np.float32)
    logits[0, 0] = row
    res = oracle.evaluate_posterior(logits, cand, retrieve, V, t, 0.09, 0.3)
    accepted = np.flatnonzero(res["path_len"][0] == 1)
    assert accepted.tolist() == ids.tolist()
    assert int(np.argmax(row)) in ids.tolist()


def test_sample_frequencies_follow_the_renormalised_set():
    rng = np.random.default_rng(11)
    row = (rng.standard_normal(60) * 2.5).astype(np.float32)
    ids, p = smp.typical_allowed(row, 0.8, 0.09, 0.3)
    w = p / p.sum()
    N = 20000
    counts = {}
    for k in range(N):
        v = smp.typical_sample(row, 0.8, 0.09, 0.3, (k + 0.5) / N)
        counts[v] = counts.get(v, 0) + 1
    assert set(counts) <= set(ids.tolist())
    for v, wv in zip(ids, w):
        assert abs(counts.get(int(v), 0) / N - wv) <= 1.0 / N + 1e-12


def test_next_token_is_drawn_at_the_last_accepted_node():
    V, T = 50, 5
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((2, T, V)) * 3).astype(np.float32)
    retrieve = np.array([[0, 1, 3], [0, 2, 4]], dtype=np.int32)
    best, acc = np.array([1, 0]), np.array([2, 1])
    got = smp.sample_next_typical(logits, retrieve, best, acc, 0.7, 0.09, 0.3, seed=5, step=9)
    u0 = smp.uniform(5, 9, 0, 0, smp.PURPOSE_NEXT_TOKEN)
    u1 = smp.uniform(5, 9, 1, 0, smp.PURPOSE_NEXT_TOKEN)
    assert got.tolist() == [smp.typical_sample(logits[0, 4], 0.7, 0.09, 0.3, u0),
                            smp.typical_sample(logits[1, 1], 0.7, 0.09, 0.3, u1)]
