"""GPU parity of medusa_build_tree against the oracle: bit-exact on every
output, the worked example, random and full trees, the largest tree, the
root alone, and every spec error with its entry index."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import tree_case, to_dev, to_host

pytestmark = pytest.mark.gpu

KIND = {"padding": 1, "empty": 2, "rank": 3, "duplicate": 4, "prefix": 5, "too_many_paths": 6}


def _gpu_tree(ch, ids, root, plen, p_max):
    out = md.medusa_build_tree(to_dev(ch), to_dev(ids), to_dev(root), to_dev(plen), p_max=p_max)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _compare(got, ref, p_max):
    for key in ("tree_candidates", "tree_indices", "parent", "depth", "position_ids", "tree_mask"):
        assert np.array_equal(got[key], ref[key]), key
    P = ref["num_paths"]
    assert int(got["num_paths"][0]) == P
    assert np.array_equal(got["retrieve"][:P], ref["retrieve"])
    assert np.all(got["retrieve"][P:] == -1)
    assert got["status"].tolist() == [0, -1]


def test_worked_example(gpu_device):
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_mask_example.json")))
    ch = np.array(g["choices"], dtype=np.int32)
    ids = np.array([g["topk_ids"]], dtype=np.int32)
    root = np.array([g["root_token"]], dtype=np.int32)
    plen = np.array([g["prefix_len"]], dtype=np.int32)
    ref = oracle.build_tree(ch, 2, 2, ids, root, plen)
    got = _gpu_tree(ch, ids, root, plen, 4)
    _compare(got, ref, 4)
    assert got["retrieve"].tolist() == g["readings"]["retrieve"]


@pytest.mark.parametrize("seed", range(6))
def test_random_trees(gpu_device, seed):
    w = synth.workload("vicuna-7b", B=3, L_range=(1, 5000))
    c = tree_case(w, seed=seed)
    got = _gpu_tree(c["choices"], c["topk_ids"], c["root"], c["prefix_len"], 64)
    _compare(got, c["ref"], 64)


def test_full_tree_tiny(gpu_device):
    w = synth.workload("tiny-f32")
    c = tree_case(w)
    got = _gpu_tree(c["choices"], c["topk_ids"], c["root"], c["prefix_len"], 8)
    _compare(got, c["ref"], 8)
    assert c["ref"]["num_paths"] == 8


def test_largest_tree(gpu_device):
    # 255 entries (T = 256), 8 heads, top-64
    w = synth.workload("vicuna-7b", B=16, K=8, topk=64, tree="random",
                       depth_counts=(40, 60, 60, 40, 25, 15, 10, 5))
    c = tree_case(w, seed=2)
    assert len(c["ref"]["nodes"]) == 256
    got = _gpu_tree(c["choices"], c["topk_ids"], c["root"], c["prefix_len"], 256)
    _compare(got, c["ref"], 256)


def test_root_only(gpu_device):
    w = synth.workload("tiny-f32")
    ch = np.zeros((0, 3), dtype=np.int32)
    ids = synth.topk_ids_input(w)
    ref = oracle.build_tree(ch, 3, 2, ids, np.array([5], np.int32), np.array([9], np.int32))
    got = _gpu_tree(ch, ids, np.array([5], np.int32), np.array([9], np.int32), 2)
    _compare(got, ref, 2)


@pytest.mark.parametrize("rows", [
    [[0, -1], [0, -1]],
    [[0, -1], [1, 0], [1, -1], [1, 0]],
    [[0, 1]],
    [[0, -1], [0, 1], [1, 1]],
    [[0, -1], [2, -1]],
    [[0, -1], [1, -5]],
    [[-1, -1]],
    [[0, -1], [-1, 1]],
    [[1, 1], [0, -1], [0, 0], [5, -1]],
])
def test_spec_errors_match_oracle(gpu_device, rows):
    ch = np.array(rows, dtype=np.int32)
    ids = np.arange(4, dtype=np.int32).reshape(1, 2, 2)
    root = np.array([7], np.int32)
    plen = np.array([3], np.int32)
    with pytest.raises(oracle.SpecError) as e:
        oracle.build_tree(ch, 2, 2, ids, root, plen)
    got = _gpu_tree(ch, ids, root, plen, 8)
    assert got["status"].tolist() == [KIND[e.value.kind], e.value.index]
    # degenerate tree: the root alone
    T = len(rows) + 1
    assert int(got["num_paths"][0]) == 1
    assert got["retrieve"][0].tolist() == [0, -1, -1]
    assert np.array_equal(got["tree_mask"], np.eye(T, dtype=np.uint8))
    assert np.all(got["tree_candidates"] == 7)


def test_too_many_paths(gpu_device):
    ch = synth.choices_array(synth.full_tree_choices(2, 3), 2)
    ids = np.zeros((1, 2, 3), dtype=np.int32)
    got = _gpu_tree(ch, ids, np.array([1], np.int32), np.array([0], np.int32), 8)
    assert got["status"].tolist() == [6, 9]
    assert int(got["num_paths"][0]) == 1


def _gather(tree, ids, root, plen):
    out = md.medusa_tree_candidates(tree["tree_indices"], tree["depth"], to_dev(ids), to_dev(root), to_dev(plen))
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


@pytest.mark.parametrize("wl,kw,p_max", [
    ("tiny-f32", {}, 8),
    ("vicuna-7b", dict(B=3, L_range=(1, 5000)), 64),
    ("vicuna-7b", dict(B=16, K=8, topk=64, tree="random", depth_counts=(40, 60, 60, 40, 25, 15, 10, 5)), 256),
])
def test_tree_candidates_gather_matches_a_full_build(gpu_device, wl, kw, p_max):
    # the tree is built once from one step's top-k; later steps' top-k, root
    # tokens and prefix lengths go through the gather, which must give the
    # candidates and positions the oracle builds from scratch for them
    w = synth.workload(wl, **kw)
    c = tree_case(w, seed=5)
    tree = md.medusa_build_tree(to_dev(c["choices"]), to_dev(c["topk_ids"]), to_dev(c["root"]),
                                to_dev(c["prefix_len"]), p_max=p_max)
    for step in range(1, 4):
        ids = synth.topk_ids_input(w, seed=5 + 100 * step)
        root = synth.root_token_input(w, seed=5 + 100 * step)
        plen = synth.prefix_lengths(w, seed=5 + 100 * step)
        ref = oracle.build_tree(c["choices"], w["K"], w["topk"], ids, root, plen)
        got = _gather(tree, ids, root, plen)
        assert np.array_equal(got["tree_candidates"], ref["tree_candidates"])
        assert np.array_equal(got["position_ids"], ref["position_ids"])


def test_tree_candidates_on_a_spec_error_tree_are_the_root(gpu_device):
    # a failed build describes the root alone (depth 0, index 0): every node
    # then gathers the root token at the prefix length
    ch = np.array([[0, -1], [0, -1]], dtype=np.int32)
    ids = np.arange(4, dtype=np.int32).reshape(1, 2, 2)
    tree = md.medusa_build_tree(to_dev(ch), to_dev(ids), to_dev(np.array([7], np.int32)),
                                to_dev(np.array([3], np.int32)), p_max=8)
    got = _gather(tree, ids + 10, np.array([9], np.int32), np.array([40], np.int32))
    assert np.all(got["tree_candidates"] == 9)
    assert np.all(got["position_ids"] == 40)


def test_tree_candidates_out_of_range_indices_read_the_root(gpu_device):
    # the header's rule: an index outside [0, 1 + K * topk) reads the root
    K, k, B = 2, 3, 2
    ids = (np.arange(B * K * k, dtype=np.int32) + 100).reshape(B, K, k)
    ti = np.array([0, 1, 6, -5, 7, 1 << 30], dtype=np.int32)
    depth = np.array([0, 1, 2, 1, 2, 3], dtype=np.int32)
    root = np.array([7, 8], dtype=np.int32)
    plen = np.array([10, 20], dtype=np.int32)
    out = md.medusa_tree_candidates(to_dev(ti), to_dev(depth), to_dev(ids), to_dev(root), to_dev(plen))
    torch.cuda.synchronize()
    cand, pos = to_host(out["tree_candidates"]), to_host(out["position_ids"])
    for b in range(B):
        flat = [root[b]] + ids[b].ravel().tolist()
        assert cand[b].tolist() == [flat[0], flat[1], flat[6], root[b], root[b], root[b]]
        assert pos[b].tolist() == (plen[b] + depth).tolist()
