"""Pins for the oracle's tree attention.

Brute force: every root-to-leaf path, appended to the prefix as an ordinary
sequence at positions L, L+1, ... and run through plain causal attention,
must give the tree output at each of its nodes (this also fixes the position
ids, since RoPE is applied at the path's sequential positions).  A one-node
tree and a chain tree reduce to PyTorch's scaled_dot_product_attention; shift
invariances and the irrelevance of non-ancestor tree rows are checked too.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _case(choices, K, topk, L, Hq, d, seed):
    rng = np.random.default_rng(seed)
    ch = synth.choices_array(choices, K)
    t = oracle.build_tree(ch, K, topk, np.zeros((1, K, topk), np.int32), np.array([0]), np.array([L]))
    T = len(t["nodes"])
    # unrotated projections for the prefix tokens and the tree tokens
    qn = rng.standard_normal((T, Hq, d))
    kp = rng.standard_normal((Hq, L, d))
    vp = rng.standard_normal((Hq, L, d))
    kn = rng.standard_normal((Hq, T, d))
    vn = rng.standard_normal((Hq, T, d))
    return t, qn, kp, vp, kn, vn


def _causal_path_outputs(path, qn, kp, vp, kn, vn, L, scale):
    """Plain causal attention over prefix + path tokens at positions L, L+1, ..."""
    Hq, _, d = kp.shape
    n = len(path)
    kp_rot = synth.rope_rotate(kp, np.arange(L))
    out = np.zeros((n, Hq, d))
    for h in range(Hq):
        keys = [kp_rot[h, m] for m in range(L)]
        vals = [vp[h, m] for m in range(L)]
        for t, node in enumerate(path):
            keys.append(synth.rope_rotate(kn[h, node][None], [L + t])[0])
            vals.append(vn[h, node])
            q = synth.rope_rotate(qn[node, h][None], [L + t])[0]
            s = [scale * float(np.dot(q, k)) for k in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = math.fsum(e)
            out[t, h] = sum(ei * v for ei, v in zip(e, vals)) / tot
    return out


def _tree_outputs(t, qn, kp, vp, kn, vn, L, scale):
    T = len(t["nodes"])
    Hq, _, d = kp.shape
    pos = L + t["depth"]
    q = synth.rope_rotate(qn.transpose(1, 0, 2), pos).transpose(1, 0, 2)[None]
    kc = np.concatenate([synth.rope_rotate(kp, np.arange(L)), synth.rope_rotate(kn, pos)], axis=1)[None]
    vc = np.concatenate([vp, vn], axis=1)[None]
    return oracle.tree_attention(q, kc, vc, np.array([L]), t["tree_mask"], scale)[0]


@pytest.mark.parametrize("spec,K,topk,seed", [
    ("worked", 2, 2, 0),
    ("full", 3, 2, 1),
    ("random", 4, 3, 2),
])
def test_tree_equals_per_path_causal(spec, K, topk, seed):
    if spec == "worked":
        choices = synth.worked_example_choices()
    elif spec == "full":
        choices = synth.full_tree_choices(K, topk)
    else:
        choices = synth.random_tree_choices((3, 4, 3, 2), topk, seed=seed)
    L, Hq, d = 5, 2, 8
    scale = 1.0 / math.sqrt(d)
    t, qn, kp, vp, kn, vn = _case(choices, K, topk, L, Hq, d, seed)
    tree = _tree_outputs(t, qn, kp, vp, kn, vn, L, scale)
    for row in t["retrieve"][:t["num_paths"]]:
        path = [int(x) for x in row if x >= 0]
        ref = _causal_path_outputs(path, qn, kp, vp, kn, vn, L, scale)
        for pos, node in enumerate(path):
            assert np.max(np.abs(tree[node] - ref[pos])) < 1e-12


def test_root_only_is_single_query_decode():
    rng = np.random.default_rng(4)
    L, Hq, d = 9, 3, 16
    q = rng.standard_normal((1, 1, Hq, d))
    kc = rng.standard_normal((1, Hq, L + 1, d))
    vc = rng.standard_normal((1, Hq, L + 1, d))
    out = oracle.tree_attention(q, kc, vc, np.array([L]), np.ones((1, 1), np.uint8), 0.37)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0].transpose(1, 0, 2)).unsqueeze(0),   # [1][Hq][1][d]
        torch.from_numpy(kc), torch.from_numpy(vc), scale=0.37)
    assert np.max(np.abs(out[0, 0] - ref[0, :, 0].numpy())) < 1e-12


def test_chain_tree_is_causal_attention():
    rng = np.random.default_rng(5)
    L, n, Hq, d = 6, 4, 2, 8
    t = oracle.build_tree(synth.choices_array(synth.chain_choices(n), n), n, 1,
                          np.zeros((1, n, 1), np.int32), np.array([0]), np.array([L]))
    T = n + 1
    q = rng.standard_normal((1, T, Hq, d))
    kc = rng.standard_normal((1, Hq, L + T, d))
    vc = rng.standard_normal((1, Hq, L + T, d))
    out = oracle.tree_attention(q, kc, vc, np.array([L]), t["tree_mask"], 0.5)
    allowed = np.concatenate([np.ones((T, L), bool), np.tril(np.ones((T, T), bool))], axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0].transpose(1, 0, 2)), torch.from_numpy(kc[0]),
        torch.from_numpy(vc[0]), attn_mask=torch.from_numpy(allowed), scale=0.5)
    assert np.max(np.abs(out[0] - ref.numpy().transpose(1, 0, 2))) < 1e-12


def test_shift_invariances_and_hidden_rows():
    w = synth.workload("tiny-f32", S_max=40)
    L, Hq, d = 20, 2, 8
    t = oracle.build_tree(synth.choices_array(synth.full_tree_choices(2, 2), 2), 2, 2,
                          np.zeros((1, 2, 2), np.int32), np.array([0]), np.array([L]))
    T = len(t["nodes"])
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, T, Hq, d))
    kc = rng.standard_normal((1, Hq, 40, d))
    vc = rng.standard_normal((1, Hq, 40, d))
    base = oracle.tree_attention(q, kc, vc, np.array([L]), t["tree_mask"], 0.3)
    # adding one vector to every key shifts all scores of a query equally
    c = rng.standard_normal(d)
    assert np.allclose(oracle.tree_attention(q, kc + c, vc, np.array([L]), t["tree_mask"], 0.3),
                       base, atol=1e-12, rtol=0)
    # adding one vector to every value shifts every output by it
    assert np.allclose(oracle.tree_attention(q, kc, vc + c, np.array([L]), t["tree_mask"], 0.3),
                       base + c, atol=1e-12, rtol=0)
    # node 3 (first child of node 1) cannot see node 2's row or slots past the tree
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, L + 2] = 1e3
    vc2[:, :, L + 2] = -7.0
    kc2[:, :, L + T:] = np.nan
    out2 = oracle.tree_attention(q, kc2, vc2, np.array([L]), t["tree_mask"], 0.3)
    assert np.array_equal(out2[0, 3], base[0, 3])
    assert not np.allclose(out2[0, 2], base[0, 2])
