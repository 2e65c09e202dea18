"""Pins for the oracle's tree builder.

The worked mask example of the study notes page (案例 3) fixes node order,
candidates and visibility; the rest are structural invariants computed
differently from the oracle (walking parent pointers instead of comparing
rank-tuple prefixes), closed-form node/path counts of full trees, and the
validator's rejections.
"""

import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_mask_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_page_facts():
    g = _golden()
    tok = g["token_ids"]
    t = oracle.build_tree(np.array(g["choices"], dtype=np.int32), g["K"], g["topk"],
                          np.array([g["topk_ids"]], dtype=np.int32),
                          np.array([g["root_token"]]), np.array([g["prefix_len"]]))
    # forward order P, A, B, X, Y, X, Y
    assert [int(x) for x in t["tree_candidates"][0]] == [tok[n] for n in g["page"]["forward_order"]]
    # each head-2 token follows the branch the page names
    names = g["page"]["forward_order"]
    for node, branch in g["page"]["branch_of"].items():
        assert names[t["parent"][int(node)]] == branch
    # each head-2 token sees exactly P and its branch token besides itself
    for node, seen in g["page"]["sees_other_than_itself"].items():
        i = int(node)
        visible = [names[j] for j in range(len(names)) if t["tree_mask"][i, j] and j != i]
        assert sorted(visible) == sorted(seen)


def test_worked_example_readings():
    g = _golden()
    r = g["readings"]
    L = g["prefix_len"]
    t = oracle.build_tree(np.array(g["choices"], dtype=np.int32), g["K"], g["topk"],
                          np.array([g["topk_ids"]], dtype=np.int32),
                          np.array([g["root_token"]]), np.array([L]))
    assert t["parent"].tolist() == r["parent"]
    assert t["depth"].tolist() == r["depth"]
    assert t["tree_indices"].tolist() == r["tree_indices"]
    assert t["retrieve"].tolist() == r["retrieve"]
    assert t["num_paths"] == len(r["retrieve"])
    assert t["position_ids"][0].tolist() == [L + o for o in r["position_offsets"]]
    T = len(r["parent"])
    want = np.zeros((T, T), dtype=np.uint8)
    for i, row in enumerate(r["mask_rows"]):
        want[i, row] = 1
    assert np.array_equal(t["tree_mask"], want)


@pytest.mark.parametrize("K,k", [(1, 1), (1, 4), (2, 2), (3, 2), (2, 3), (3, 3), (4, 2)])
def test_full_tree_counts(K, k):
    ch = synth.choices_array(synth.full_tree_choices(K, k), K)
    ids = np.arange(K * k, dtype=np.int32).reshape(1, K, k) + 1000
    t = oracle.build_tree(ch, K, k, ids, np.array([7]), np.array([0]))
    T = sum(k ** i for i in range(K + 1))
    assert len(t["nodes"]) == T
    assert t["num_paths"] == k ** K
    assert t["retrieve"].shape == (k ** K, K + 1)
    assert np.all(t["retrieve"] >= 0)          # every leaf is at full depth
    # the leaves' rank tuples are every tuple of length K exactly once
    leaves = {t["nodes"][row[-1]] for row in t["retrieve"]}
    assert len(leaves) == k ** K


def _walk_ancestors(parent, i):
    out = {i}
    while parent[i] >= 0:
        i = int(parent[i])
        out.add(i)
    return out


def _check_invariants(t, K, topk, topk_ids, root, L):
    T = len(t["nodes"])
    parent, depth, mask = t["parent"], t["depth"], t["tree_mask"]
    assert parent[0] == -1 and depth[0] == 0
    for i in range(1, T):
        assert 0 <= parent[i] < i
        assert depth[i] == depth[parent[i]] + 1
        assert depth[i] >= depth[i - 1]           # nodes grouped by depth
    assert np.array_equal(mask, np.tril(mask))
    assert np.all(np.diag(mask) == 1)
    assert np.array_equal(mask.sum(axis=1), depth + 1)
    for i in range(T):
        anc = _walk_ancestors(parent, i)
        assert set(np.flatnonzero(mask[i]).tolist()) == anc
    # candidates: token of head depth-1 at the node's own rank
    for b in range(topk_ids.shape[0]):
        assert t["tree_candidates"][b, 0] == root[b]
        for i in range(1, T):
            rank = t["nodes"][i][-1]
            assert t["tree_candidates"][b, i] == topk_ids[b, depth[i] - 1, rank]
            assert t["tree_indices"][i] - 1 == (depth[i] - 1) * topk + rank
        assert np.array_equal(t["position_ids"][b], L[b] + depth)
    # paths: root-to-leaf along parent pointers, every leaf once, covering all nodes
    children = np.zeros(T, dtype=int)
    for i in range(1, T):
        children[parent[i]] += 1
    leaves = [i for i in range(T) if children[i] == 0]
    P = t["num_paths"]
    assert P == len(leaves)
    covered = set()
    for p in range(P):
        row = [int(x) for x in t["retrieve"][p] if x >= 0]
        assert row[0] == 0 and row[-1] == leaves[p]
        for a, c in zip(row, row[1:]):
            assert parent[c] == a
        assert all(x == -1 for x in t["retrieve"][p][len(row):])
        covered.update(row)
    assert covered == set(range(T))


@pytest.mark.parametrize("seed", range(12))
def test_random_tree_invariants(seed):
    w = synth.workload("vicuna-7b")
    choices = synth.random_tree_choices(w["depth_counts"], w["topk"], seed=seed, workload_id=w["wid"])
    ch = synth.choices_array(choices, w["K"])
    ids = synth.topk_ids_input(dict(w, B=2), seed=seed)
    root = np.array([5, 9])
    L = np.array([100, 2048])
    t = oracle.build_tree(ch, w["K"], w["topk"], ids, root, L)
    assert len(t["nodes"]) == 64
    assert np.bincount(t["depth"]).tolist() == [1, 10, 20, 16, 10, 7]
    _check_invariants(t, w["K"], w["topk"], ids, root, L)


@pytest.mark.parametrize("K,k", [(3, 2), (2, 3)])
def test_full_tree_invariants(K, k):
    ch = synth.choices_array(synth.full_tree_choices(K, k), K)
    ids = np.random.default_rng(3).integers(0, 50, size=(1, K, k)).astype(np.int32)
    _check_invariants(oracle.build_tree(ch, K, k, ids, np.array([1]), np.array([4])),
                      K, k, ids, np.array([1]), np.array([4]))


def test_spec_order_does_not_matter():
    w = synth.workload("vicuna-7b")
    a = synth.random_tree_choices(w["depth_counts"], w["topk"], seed=1, shuffle=False)
    b = list(reversed(a))
    ids = synth.topk_ids_input(w, seed=1)
    ta = oracle.build_tree(synth.choices_array(a, 5), 5, 10, ids, np.array([3]), np.array([9]))
    tb = oracle.build_tree(synth.choices_array(b, 5), 5, 10, ids, np.array([3]), np.array([9]))
    for key in ("tree_candidates", "tree_indices", "parent", "depth", "position_ids",
                "tree_mask", "retrieve"):
        assert np.array_equal(ta[key], tb[key])


def test_chain_and_root_only():
    ch = synth.choices_array(synth.chain_choices(4), 4)
    ids = np.zeros((1, 4, 1), dtype=np.int32)
    t = oracle.build_tree(ch, 4, 1, ids, np.array([1]), np.array([0]))
    assert t["retrieve"].tolist() == [[0, 1, 2, 3, 4]]
    assert np.array_equal(t["tree_mask"], np.tril(np.ones((5, 5), dtype=np.uint8)))
    t0 = oracle.build_tree(np.zeros((0, 3), dtype=np.int32), 3, 2, np.zeros((1, 3, 2), np.int32),
                           np.array([4]), np.array([10]))
    assert t0["retrieve"].tolist() == [[0, -1, -1, -1]]
    assert t0["tree_candidates"].tolist() == [[4]]


@pytest.mark.parametrize("rows,kind", [
    ([[0, -1], [0, -1]], "duplicate"),
    ([[0, 1]], "prefix"),
    ([[0, -1], [2, -1]], "rank"),
    ([[0, -1], [-3, -1]], "rank"),
    ([[-1, -1]], "empty"),
    ([[-1, 0]], "padding"),
])
def test_validator_rejects(rows, kind):
    with pytest.raises(oracle.SpecError) as e:
        oracle.build_tree(np.array(rows, dtype=np.int32), 2, 2, np.zeros((1, 2, 2), np.int32),
                          np.array([0]), np.array([0]))
    assert e.value.kind == kind


def test_too_many_paths():
    ch = synth.choices_array(synth.full_tree_choices(2, 3), 2)
    with pytest.raises(oracle.SpecError) as e:
        oracle.build_tree(ch, 2, 3, np.zeros((1, 2, 3), np.int32), np.array([0]), np.array([0]),
                          p_max=8)
    assert e.value.kind == "too_many_paths"
