"""GPU parity at the tree shapes the tree-shape sweep times (Vicuna-7B
sizes, batch 1): heads with K = 3, 4 and 8 (K = 5 is the main heads case),
and for every swept (K, T) the best-first tree of T nodes under the
synthetic acceptance model -- its build bit-exact, tree attention at 32 x 128
heads over a 2048-token prefix within 2e-2, greedy and typical acceptance on
planted logits bit-exact, and the commit of the deepest path byte-exact."""

import math

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import heads_case, posterior_case, rel_err, tol, to_dev, to_host, tree_case

pytestmark = pytest.mark.gpu

SWEEP_K = (3, 4, 5, 8)
SWEEP_T = (16, 32, 64, 128)


@pytest.mark.parametrize("K", [3, 4, 8])
def test_heads_vicuna7b_head_counts(gpu_device, K):
    # the swept head counts at H 4096, V 32000 (the workgroups per head
    # change with K); the row-major two-call form the sweep times
    w = synth.workload("vicuna-7b", K=K)
    case = heads_case(w, seed=K)
    x = case["inputs"]
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    r = md.medusa_resblock(h, w1, b1)
    out = md.medusa_lm_head_topk(r, wlm, w["topk"])
    torch.cuda.synchronize()
    print("K", K, "retries", case["retries"], flush=True)
    assert rel_err(to_host(r), case["r"]) < tol("bf16")
    assert np.array_equal(to_host(out["topk_ids"]), case["topk_ids"])
    assert rel_err(to_host(out["topk_logits"]), case["topk_logits"]) < tol("bf16")


_TREES = {}


def _sweep_tree(K, T):
    """Workload and tree case of one swept shape (cached)."""
    if (K, T) not in _TREES:
        w = synth.workload("vicuna-7b", K=K, S_max=2048 + max(SWEEP_T) + 8)
        choices = synth.best_tree_choices(synth.geometric_acceptance(K, w["topk"]), T - 1)
        _TREES[(K, T)] = (w, tree_case(w, seed=K * 1000 + T, choices=choices))
    return _TREES[(K, T)]


@pytest.mark.parametrize("T", SWEEP_T)
@pytest.mark.parametrize("K", SWEEP_K)
def test_sweep_tree_build(gpu_device, K, T):
    w, c = _sweep_tree(K, T)
    ref = c["ref"]
    assert len(ref["nodes"]) == T
    out = md.medusa_build_tree(to_dev(c["choices"]), to_dev(c["topk_ids"]), to_dev(c["root"]),
                               to_dev(c["prefix_len"]), p_max=T)
    torch.cuda.synchronize()
    got = {k: to_host(v) for k, v in out.items()}
    for key in ("tree_candidates", "tree_indices", "parent", "depth", "position_ids", "tree_mask"):
        assert np.array_equal(got[key], ref[key]), key
    P = ref["num_paths"]
    assert int(got["num_paths"][0]) == P
    assert np.array_equal(got["retrieve"][:P], ref["retrieve"])
    assert got["status"].tolist() == [0, -1]


@pytest.mark.parametrize("T", SWEEP_T)
@pytest.mark.parametrize("K", SWEEP_K)
def test_sweep_tree_attention(gpu_device, K, T):
    w, c = _sweep_tree(K, T)
    ref_tree = c["ref"]
    plen = c["prefix_len"]
    x = synth.attention_inputs(w, ref_tree["depth"], plen, seed=K + T)
    scale = 1.0 / math.sqrt(w["d"])
    ref = oracle.tree_attention(x["q"], x["k_cache"], x["v_cache"], plen, ref_tree["tree_mask"], scale)
    out = md.medusa_tree_attention(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(plen),
                                   to_dev(ref_tree["tree_mask"]), scale)
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(to_host(out))
    assert not np.any(np.isnan(got))
    err = rel_err(got, ref)
    print("K", K, "T", T, "attention max rel err %.3e" % err, flush=True)
    assert err < tol("bf16")


@pytest.mark.parametrize("temperature", [0.0, 0.7])
@pytest.mark.parametrize("T", SWEEP_T)
@pytest.mark.parametrize("K", SWEEP_K)
def test_sweep_posterior_and_commit(gpu_device, K, T, temperature):
    w, c = _sweep_tree(K, T)
    t = c["ref"]
    pc = posterior_case(w, c, temperature, seed=K + T)
    post = md.medusa_evaluate_posterior(to_dev(pc["logits"]), to_dev(t["tree_candidates"]), to_dev(t["retrieve"]),
                                        to_dev(np.array([t["num_paths"]], dtype=np.int32)), temperature, w["eps"],
                                        w["delta"])
    torch.cuda.synchronize()
    exp = pc["ref"]
    for key in ("best_path", "accept_len", "next_token"):
        assert to_host(post[key]).tolist() == exp[key].tolist(), key
    # commit the accepted path over four layers of the 32-head cache
    nl, S = 4, w["S_max"]
    g = np.random.default_rng(K * T)
    kc = g.integers(0, 1 << 16, size=(nl, 1, w["Hq"], S, w["d"]), dtype=np.uint16)
    vc = g.integers(0, 1 << 16, size=(nl, 1, w["Hq"], S, w["d"]), dtype=np.uint16)
    ek, ev, elen = oracle.commit_kv(kc, vc, c["prefix_len"], t["retrieve"], exp["best_path"], exp["accept_len"])
    dk, dv = to_dev(kc), to_dev(vc)
    newlen = md.medusa_commit_kv(dk, dv, to_dev(c["prefix_len"]), to_dev(t["retrieve"]), post["best_path"],
                                 post["accept_len"])
    torch.cuda.synchronize()
    assert to_host(newlen).tolist() == elen.tolist()
    assert np.array_equal(to_host(dk).view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(to_host(dv).view(np.uint8), ev.view(np.uint8))
