"""GPU parity of medusa_heads_tree: the Medusa heads and the per-step tree
gather in one call, against the oracle.

Top-k ids are compared bit for bit with the oracle's (inputs redrawn until
the oracle's top-k gaps clear float error), top-k logits within the float
bar, and tree_candidates / position_ids bit for bit with the oracle's tree
built on the oracle's top-k.  Every case also equals medusa_heads followed
by medusa_tree_candidates on the same inputs.  Paths: the gather inside the
lm_head kernel (bf16, batch <= 2, in-kernel merge: the Vicuna-7B shape with
its 64-node tree, and K = 8), the separate merge kernel followed by the
gather launch (K = 2 with top-10, batch 2), the skinny-GEMM path (batch 3),
the float32 kernels, a root-only tree, and calls in turn on one workspace
with different inputs.
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import heads_case, rel_err, to_dev, to_host, tol, tree_spec

pytestmark = pytest.mark.gpu


def _tree_inputs(w, seed, choices):
    ch = synth.choices_array(choices, w["K"])
    root = synth.root_token_input(w, seed=seed)
    plen = synth.prefix_lengths(w, seed=seed)
    # tree_indices and depth of the spec (they do not depend on the top-k)
    shape = oracle.build_tree(ch, w["K"], w["topk"], np.zeros((w["B"], w["K"], w["topk"]), np.int32), root, plen)
    return ch, root, plen, shape


def _run(case, w, seed, choices, ws=None):
    x = case["inputs"]
    ch, root, plen, shape = _tree_inputs(w, seed, choices)
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    tidx, dep = to_dev(shape["tree_indices"].astype(np.int32)), to_dev(shape["depth"].astype(np.int32))
    rt, pl = to_dev(root), to_dev(plen)
    got = md.medusa_heads_tree(h, w1, b1, wlm, w["topk"], tidx, dep, rt, pl, ws=ws)
    # the same work as two calls
    two = md.medusa_heads(h, w1, b1, wlm, w["topk"], ws=ws)
    tc = md.medusa_tree_candidates(tidx, dep, two["topk_ids"], rt, pl)
    torch.cuda.synchronize()
    ref = oracle.build_tree(ch, w["K"], w["topk"], case["topk_ids"], root, plen)
    return {k: to_host(v) for k, v in got.items() if v is not None}, two, tc, ref


def _check(case, w, seed, choices, ws=None):
    got, two, tc, ref = _run(case, w, seed, choices, ws)
    print("retries", case["retries"], "T", ref["tree_candidates"].shape[1], flush=True)
    assert np.array_equal(got["topk_ids"], case["topk_ids"])
    assert rel_err(got["topk_logits"], case["topk_logits"]) < tol(w["dtype"])
    assert np.array_equal(got["tree_candidates"], ref["tree_candidates"])
    assert np.array_equal(got["position_ids"], ref["position_ids"])
    assert np.array_equal(got["topk_ids"], to_host(two["topk_ids"]))
    assert np.array_equal(got["topk_logits"], to_host(two["topk_logits"]))
    assert np.array_equal(got["tree_candidates"], to_host(tc["tree_candidates"]))
    assert np.array_equal(got["position_ids"], to_host(tc["position_ids"]))
    return got


def _random_choices(K, topk, seed):
    counts = [min(topk, 6)] + [max(1, 10 - 2 * d) for d in range(1, K)]
    return synth.random_tree_choices(counts, topk, seed=seed)


def test_heads_tree_vicuna7b(gpu_device):
    # K 5, top-10, 64-node tree: the gather inside the lm_head kernel
    w = synth.workload("vicuna-7b")
    case = heads_case(w, seed=3)
    _check(case, w, 3, tree_spec(w, 3))


@pytest.mark.parametrize("B,H,V,K,k", [
    (1, 1024, 5000, 8, 8),     # in-kernel merge and gather, eight heads
    (2, 520, 3001, 2, 10),     # batch 2, separate merge kernel, then the gather launch
    (3, 264, 2000, 3, 5),      # batch 3: skinny-GEMM path, merge kernel, gather launch
])
def test_heads_tree_paths(gpu_device, B, H, V, K, k):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=B + K, margin=1e-5, max_retries=400)
    _check(case, w, B + K, _random_choices(K, k, B * K))


def test_heads_tree_f32(gpu_device):
    w = synth.workload("tiny-f32", B=2, H=132, V=333, K=3, topk=6)
    case = heads_case(w, seed=4)
    _check(case, w, 4, _random_choices(3, 6, 4))


def test_heads_tree_root_only(gpu_device):
    # an empty spec: one node, the root token at prefix_len + 0
    w = synth.workload("vicuna-7b", B=1, H=512, V=4000, K=5, topk=10)
    case = heads_case(w, seed=9, margin=1e-5, max_retries=400)
    got = _check(case, w, 9, [])
    assert got["tree_candidates"].shape == (1, 1)


def test_heads_tree_calls_in_turn_share_workspace(gpu_device):
    # different inputs in turn (A, B, A, B) on one workspace: the head and
    # gather arrival counts are left at zero by every call, and each gather
    # reads the running call's top-k
    w = synth.workload("vicuna-7b", B=1, H=512, V=6000, K=5, topk=10)
    a = heads_case(w, seed=21)
    b = heads_case(w, seed=22)
    assert not np.array_equal(a["topk_ids"], b["topk_ids"])
    ws = torch.zeros(md.medusa_heads_workspace(md.MEDUSA_BF16, 1, 512, 6000, 5, 10), dtype=torch.uint8,
                     device=gpu_device)
    spec = _random_choices(5, 10, 7)
    for case, seed in ((a, 21), (b, 22), (a, 21), (b, 22)):
        _check(case, w, seed, spec, ws=ws)


def test_lm_head_topk_tree_split_form(gpu_device):
    # medusa_resblock, then medusa_lm_head_topk_tree (the bench's step) at
    # the Vicuna-7B shape and 64-node tree
    w = synth.workload("vicuna-7b")
    case = heads_case(w, seed=5)
    x = case["inputs"]
    ch, root, plen, shape = _tree_inputs(w, 5, tree_spec(w, 5))
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    tidx, dep = to_dev(shape["tree_indices"].astype(np.int32)), to_dev(shape["depth"].astype(np.int32))
    r = md.medusa_resblock(h, w1, b1)
    for _ in range(2):
        got = md.medusa_lm_head_topk_tree(r, wlm, w["topk"], tidx, dep, to_dev(root), to_dev(plen))
        torch.cuda.synchronize()
        ref = oracle.build_tree(ch, w["K"], w["topk"], case["topk_ids"], root, plen)
        assert np.array_equal(to_host(got["topk_ids"]), case["topk_ids"])
        assert rel_err(to_host(got["topk_logits"]), case["topk_logits"]) < tol(w["dtype"])
        assert np.array_equal(to_host(got["tree_candidates"]), ref["tree_candidates"])
        assert np.array_equal(to_host(got["position_ids"]), ref["position_ids"])
