"""Pins for the oracle's nucleus (top-p) acceptance.

Each check stands outside the oracle's own code:
  * a four-token case worked by hand (probabilities 0.1, 0.4, 0.2, 0.3);
  * tiny top_p: the nucleus is the argmax alone (np.argmax, first maximum),
    whatever the uniform;
  * equal logits: ties go to the lower token id (top_p 0.45 of ten equal
    tokens keeps ids 0..4);
  * the nucleus's defining properties on random rows: it reaches top_p,
    every token outside is no more likely than every token inside, and
    without its least likely member it falls short of top_p;
  * inverse-CDF sampling over a uniform grid of u reproduces the
    renormalised nucleus probabilities to within one grid step, and never
    returns a token outside the nucleus;
  * acceptance on the worked tree: with one-hot rows it equals greedy
    acceptance (pinned on its own); with two-token nuclei the uniforms
    decide which child survives, as worked by hand.
"""

import numpy as np
import pytest

import oracle


def _logits_for(p):
    return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


def test_hand_worked_four_tokens():
    x = _logits_for([0.1, 0.4, 0.2, 0.3])
    # descending: 1 (0.4), 3 (0.3), 2 (0.2), 0 (0.1); masses 0.4, 0.7, ...
    ids, p = oracle.nucleus(x, 1.0, 0.65)
    assert ids.tolist() == [1, 3]
    assert np.allclose(p, [0.4, 0.3], rtol=1e-6)
    ids, _ = oracle.nucleus(x, 1.0, 0.35)
    assert ids.tolist() == [1]
    ids, _ = oracle.nucleus(x, 1.0, 0.75)
    assert ids.tolist() == [1, 2, 3]
    # sampling in id order over {1, 3}, mass 0.7: u 0.5 -> 0.35 < 0.4 -> 1;
    # u 0.6 -> 0.42 -> token 3; u 0 -> first id
    assert oracle.nucleus_sample(x, 1.0, 0.65, 0.5) == 1
    assert oracle.nucleus_sample(x, 1.0, 0.65, 0.6) == 3
    assert oracle.nucleus_sample(x, 1.0, 0.65, 0.0) == 1
    assert oracle.nucleus_sample(x, 1.0, 0.65, 0.999) == 3


def test_tiny_top_p_is_argmax():
    rng = np.random.default_rng(1)
    for _ in range(20):
        x = (rng.standard_normal(300) * 3).astype(np.float32)
        x[rng.integers(300)] = x.max()          # a tied maximum now and then
        for u in (0.0, 0.3, 0.99):
            assert oracle.nucleus_sample(x, 0.7, 1e-7, u) == int(np.argmax(x))


def test_ties_take_lower_ids():
    x = np.zeros(10, dtype=np.float32)
    ids, p = oracle.nucleus(x, 1.0, 0.45)
    assert ids.tolist() == [0, 1, 2, 3, 4]
    assert np.allclose(p, 0.1)
    ids, _ = oracle.nucleus(x, 1.0, 1.0)
    assert ids.tolist() == list(range(10))


@pytest.mark.parametrize("seed", range(6))
def test_nucleus_defining_properties(seed):
    rng = np.random.default_rng(seed)
    V = 500
    x = (rng.standard_normal(V) * (1 + seed)).astype(np.float32)
    t, q = 0.7, float(np.float32(0.8))
    z = x.astype(np.float64) / float(np.float32(t))
    full = np.exp(z - z.max())
    full /= full.sum()
    ids, p = oracle.nucleus(x, t, q)
    assert np.allclose(p, full[ids], rtol=1e-12)
    inside = np.zeros(V, dtype=bool)
    inside[ids] = True
    assert p.sum() >= q - 1e-12
    if (~inside).any():
        assert full[~inside].max() <= full[inside].min()
    assert p.sum() - p.min() < q


@pytest.mark.parametrize("top_p", [0.3, 0.8, 1.0])
def test_sampling_reproduces_nucleus_probabilities(top_p):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(40) * 1.5).astype(np.float32)
    ids, p = oracle.nucleus(x, 1.0, top_p)
    N = 4000
    counts = {}
    for i in range(N):
        s = oracle.nucleus_sample(x, 1.0, top_p, (i + 0.5) / N)
        counts[s] = counts.get(s, 0) + 1
    assert set(counts) <= set(ids.tolist())
    for v, pv in zip(ids.tolist(), p / p.sum()):
        assert abs(counts.get(v, 0) / N - pv) <= 1.0 / N + 1e-12


def _worked_tree():
    # root 0; depth-1 nodes 1 (token 10), 2 (token 11); node 3 (token 20)
    # under 1, node 4 (token 21) under 2.  Paths: 0-1-3, 0-2-4.
    cand = np.array([[5, 10, 11, 20, 21]], dtype=np.int32)
    retrieve = np.array([[0, 1, 3], [0, 2, 4]], dtype=np.int32)
    return cand, retrieve


def test_one_hot_rows_equal_greedy_acceptance():
    cand, retrieve = _worked_tree()
    V = 32
    rng = np.random.default_rng(3)
    for trial in range(10):
        top = rng.integers(V, size=5)
        x = np.full((1, 5, V), -30.0, dtype=np.float32)
        x[0, np.arange(5), top] = 10.0
        u = rng.random((1, 5)).astype(np.float32)
        got = oracle.evaluate_posterior_nucleus(x, cand, retrieve, 2, 1.0, 0.8, u)
        ref = oracle.evaluate_posterior(x, cand, retrieve, 2, 0.0, 0.09, 0.3)
        for key in ("best_path", "accept_len", "next_token"):
            assert np.array_equal(got[key], ref[key]), (trial, key)
        assert got["samples"][0].tolist() == top.tolist()


def test_uniforms_choose_between_two_token_nuclei():
    cand, retrieve = _worked_tree()
    V = 32
    x = np.full((1, 5, V), -40.0, dtype=np.float32)
    # root: tokens 10 and 11 at 0.5 each (ids ascending: 10 first)
    x[0, 0, 10] = x[0, 0, 11] = 0.0
    # node 1: token 20 (0.6) and 3 (0.4); node 2: token 21 only
    x[0, 1, 20], x[0, 1, 3] = np.log(0.6), np.log(0.4)
    x[0, 2, 21] = 0.0
    x[0, 3, 7] = x[0, 4, 9] = 0.0
    # u(root) 0.2 -> token 10 (node 1); u(node 1) 0.5 -> 0.5 in id order
    # {3: 0.4, 20: 0.6} -> running 0.4, 1.0 -> token 20 (node 3): path 0
    # accepts 2, next token = sample at node 3 = 7
    u = np.array([[0.2, 0.5, 0.0, 0.0, 0.0]], dtype=np.float32)
    got = oracle.evaluate_posterior_nucleus(x, cand, retrieve, 2, 1.0, 0.95, u)
    assert (got["best_path"][0], got["accept_len"][0], got["next_token"][0]) == (0, 2, 7)
    # u(node 1) 0.3 -> token 3: node 3 rejected; path 0 and path 1 tie? no:
    # root sample is 10, so path 1 rejects at once; path 0 accepts 1, next 3
    u[0, 1] = 0.3
    got = oracle.evaluate_posterior_nucleus(x, cand, retrieve, 2, 1.0, 0.95, u)
    assert (got["best_path"][0], got["accept_len"][0], got["next_token"][0]) == (0, 1, 3)
    # u(root) 0.7 -> token 11: path 1 accepts node 2, then 21 -> node 4: 2
    u[0, 0] = 0.7
    got = oracle.evaluate_posterior_nucleus(x, cand, retrieve, 2, 1.0, 0.95, u)
    assert (got["best_path"][0], got["accept_len"][0], got["next_token"][0]) == (1, 2, 9)


def test_rejects_bad_parameters():
    x = np.zeros(4, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.nucleus(x, 0.0, 0.8)
    with pytest.raises(ValueError):
        oracle.nucleus(x, 1.0, 0.0)
    with pytest.raises(ValueError):
        oracle.nucleus(x, 1.0, 1.5)
