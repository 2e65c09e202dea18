"""The synthetic acceptance model behind the tree-shape sweep (host logic).

best_tree_choices must return the n most probable rank tuples (checked
against sorting every tuple of a small (K, topk) by brute force), form a
valid tree (every tuple's ancestors chosen) and come out in non-increasing
probability.  expected_accept_length must equal the mean accepted length
obtained by enumerating every outcome of the model exactly: at each depth
the base model's token is head d's rank i with chance p[d][i], or none of
the head's candidates; a step accepts the longest prefix of those ranks
that is a path of the tree.
"""

import itertools

import numpy as np
import pytest

import synth


def _all_tuples(K, topk):
    return [t for d in range(1, K + 1) for t in itertools.product(range(topk), repeat=d)]


@pytest.mark.parametrize("K,topk,n", [(3, 3, 1), (3, 3, 7), (3, 3, 39), (2, 4, 11), (4, 2, 20)])
def test_best_tree_is_the_n_most_probable_tuples(K, topk, n):
    p = synth.geometric_acceptance(K, topk, q1=0.8, gamma=0.7, rho=0.3)
    got = synth.best_tree_choices(p, n)
    assert len(got) == n == len(set(got))
    probs = [synth.path_probability(p, t) for t in got]
    assert all(a >= b for a, b in zip(probs, probs[1:]))
    allp = sorted((synth.path_probability(p, t) for t in _all_tuples(K, topk)), reverse=True)
    assert np.allclose(sorted(probs, reverse=True), allp[:n], rtol=0, atol=1e-15)
    chosen = set(got)
    for t in got:
        for d in range(1, len(t)):
            assert t[:d] in chosen


def test_best_tree_rejects_too_many_nodes():
    p = synth.geometric_acceptance(2, 2)
    with pytest.raises(ValueError):
        synth.best_tree_choices(p, 7)


def test_geometric_acceptance_values():
    p = synth.geometric_acceptance(3, 4, q1=0.8, gamma=0.5, rho=0.25)
    assert p.shape == (3, 4)
    assert p[0, 0] == pytest.approx(0.8 * 0.75)
    assert p[2, 1] == pytest.approx(0.8 * 0.25 * 0.75 * 0.25)
    # each head's chance over its ranks stays below q1 gamma^d
    assert np.all(p.sum(axis=1) < 0.8 * 0.5 ** np.arange(3))


@pytest.mark.parametrize("choices", [
    [(0,)],
    [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)],
    [(0,), (0, 0), (0, 0, 0), (2,), (0, 2), (2, 1)],
])
def test_expected_accept_length_by_exact_enumeration(choices):
    K, topk = 3, 3
    p = synth.geometric_acceptance(K, topk, q1=0.9, gamma=0.8, rho=0.4)
    tree = set(choices)
    # outcome per depth: rank 0..topk-1, or topk = no candidate of that head
    mean = 0.0
    for outcome in itertools.product(range(topk + 1), repeat=K):
        prob = 1.0
        for d, o in enumerate(outcome):
            prob *= p[d][o] if o < topk else 1.0 - p[d].sum()
        acc = 0
        while acc < K and outcome[acc] < topk and tuple(outcome[:acc + 1]) in tree:
            acc += 1
        mean += prob * acc
    assert synth.expected_accept_length(p, choices) == pytest.approx(mean, rel=1e-12)
