"""HIP-graph capture of a whole verify step: every replay equals the eager step.

The library only launches kernels on the caller's stream (no allocation,
memset or synchronisation inside a call), so one verify step (heads, tree,
one attention layer, posterior, commit) captures into a single graph.  The
graph is replayed several times; between replays eager work poisons every
output and restores the in-place KV caches, with synchronisations around
each replay, and every output of every replay must equal the eager step's
bit for bit (the kernels are deterministic).  Three steps: batch 1 with
row-major heads and a full tree build, batch 4 with packed heads (the
sliced ResBlock GEMM, its finisher, the lm_head GEMM and the merge) and the
per-step tree gather on a tree built before capture, and batch 1 with the
gather inside the lm_head kernel (medusa_lm_head_topk_tree, whose arrival
counts every replay must find at zero and leave at zero).
"""

import pytest
import torch

import speculative_decoding_medusa_amd as md
import synth


def _setup(dev, B=1):
    g = torch.Generator().manual_seed(11 + B)
    H, V, K, k = 1024, 3000, 3, 4
    Hq, d, L, NL = 4, 128, 300, 2
    choices = synth.choices_array(synth.random_tree_choices([4, 6, 5], k, seed=1), K)
    T = choices.shape[0] + 1
    S = L + T + 8
    bf = torch.bfloat16
    x = dict(
        hidden=torch.randn(B, H, generator=g).to(bf).to(dev),
        w1=(torch.randn(K, H, H, generator=g) * 0.02).to(bf).to(dev),
        b1=(torch.randn(K, H, generator=g) * 0.02).to(bf).to(dev),
        w_lm=(torch.randn(K, V, H, generator=g) * 0.02).to(bf).to(dev),
        choices=torch.from_numpy(choices).to(dev),
        root=torch.tensor([5 + 7 * b for b in range(B)], dtype=torch.int32, device=dev),
        plen=torch.tensor([L - 37 * b for b in range(B)], dtype=torch.int32, device=dev),
        q=torch.randn(B, T, Hq, d, generator=g).to(bf).to(dev),
        kc0=torch.randn(NL, B, Hq, S, d, generator=g).to(bf).to(dev),
        vc0=torch.randn(NL, B, Hq, S, d, generator=g).to(bf).to(dev),
        logits=(torch.randn(B, T, V, generator=g) * 4).to(dev),
    )
    i32, f32 = torch.int32, torch.float32
    o = dict(
        r=torch.empty(B, K, H, dtype=f32, device=dev),
        heads=dict(topk_ids=torch.empty(B, K, k, dtype=i32, device=dev),
                   topk_logits=torch.empty(B, K, k, dtype=f32, device=dev)),
        tree=dict(tree_candidates=torch.empty(B, T, dtype=i32, device=dev),
                  tree_indices=torch.empty(T, dtype=i32, device=dev),
                  parent=torch.empty(T, dtype=i32, device=dev), depth=torch.empty(T, dtype=i32, device=dev),
                  position_ids=torch.empty(B, T, dtype=i32, device=dev),
                  tree_mask=torch.empty(T, T, dtype=torch.uint8, device=dev),
                  retrieve=torch.empty(T, K + 1, dtype=i32, device=dev),
                  num_paths=torch.empty(1, dtype=i32, device=dev), status=torch.empty(2, dtype=i32, device=dev)),
        att=torch.empty(B, T, Hq, d, dtype=bf, device=dev),
        post=dict(best_path=torch.empty(B, dtype=i32, device=dev), accept_len=torch.empty(B, dtype=i32, device=dev),
                  next_token=torch.empty(B, dtype=i32, device=dev)),
        new_plen=torch.empty(B, dtype=i32, device=dev),
        kc=x["kc0"].clone(), vc=x["vc0"].clone(),
        ws_h=torch.zeros(md.medusa_heads_workspace(md.MEDUSA_BF16, B, H, V, K, k), dtype=torch.uint8, device=dev),
        ws_a=torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, B, T, Hq, d, S), dtype=torch.uint8,
                         device=dev),
        ws_p=torch.zeros(md.medusa_posterior_workspace(B, T, V), dtype=torch.uint8, device=dev),
    )
    x["w1_packed"] = md.medusa_heads_pack(x["w1"])
    x["w_lm_packed"] = md.medusa_heads_pack(x["w_lm"])
    return x, o, k, d


def _step(x, o, k, d, packed=False, fused=False):
    t = o["tree"]
    if fused:   # the bench's step: the gather in the lm_head kernel's tail
        md.medusa_resblock(x["hidden"], x["w1"], x["b1"], r=o["r"])
        md.medusa_lm_head_topk_tree(o["r"], x["w_lm"], k, t["tree_indices"], t["depth"], x["root"], x["plen"],
                                    out=dict(o["heads"], tree_candidates=t["tree_candidates"],
                                             position_ids=t["position_ids"]), ws=o["ws_h"])
    elif packed:
        md.medusa_heads_packed(x["hidden"], x["w1_packed"], x["b1"], x["w_lm_packed"], x["w_lm"].shape[1], k,
                               keep_r=True, out=dict(o["heads"], r=o["r"]), ws=o["ws_h"])
        md.medusa_tree_candidates(t["tree_indices"], t["depth"], o["heads"]["topk_ids"], x["root"], x["plen"], out=t)
    else:
        md.medusa_resblock(x["hidden"], x["w1"], x["b1"], r=o["r"])
        md.medusa_lm_head_topk(o["r"], x["w_lm"], k, out=o["heads"], ws=o["ws_h"])
        md.medusa_build_tree(x["choices"], o["heads"]["topk_ids"], x["root"], x["plen"],
                             p_max=t["retrieve"].shape[0], out=t)
    md.medusa_tree_attention(x["q"], o["kc"][0], o["vc"][0], x["plen"], t["tree_mask"], d ** -0.5, out=o["att"],
                             ws=o["ws_a"])
    md.medusa_evaluate_posterior(x["logits"], t["tree_candidates"], t["retrieve"], t["num_paths"], 0.7, 0.09, 0.3,
                                 out=o["post"], ws=o["ws_p"])
    md.medusa_commit_kv(o["kc"], o["vc"], x["plen"], t["retrieve"], o["post"]["best_path"], o["post"]["accept_len"],
                        new_prefix_len=o["new_plen"])


PER_STEP_TREE = ("tree_candidates", "position_ids")


def _outputs(o, gather=False):
    """Every output of a step (with the per-step gather, the tree's own
    buffers are inputs built once, so only its candidates and positions)."""
    out = {"r": o["r"], "att": o["att"], "new_plen": o["new_plen"], "kc": o["kc"], "vc": o["vc"]}
    for grp in ("heads", "tree", "post"):
        for n, tns in o[grp].items():
            if gather and grp == "tree" and n not in PER_STEP_TREE:
                continue
            out[grp + "." + n] = tns
    return out


def _reset(x, o, gather=False):
    """Eager work between replays: poison every output, restore the caches."""
    for n, tns in _outputs(o, gather).items():
        if n in ("kc", "vc"):
            continue
        if tns.dtype.is_floating_point:
            tns.fill_(float("nan"))
        else:
            tns.fill_(-7)
    o["kc"].copy_(x["kc0"])
    o["vc"].copy_(x["vc0"])


@pytest.mark.gpu
@pytest.mark.parametrize("B,packed,fused", [(1, False, False), (4, True, False), (1, False, True)])
def test_step_graph_replays_equal_eager(gpu_device, B, packed, fused):
    x, o, k, d = _setup(gpu_device, B)
    t = o["tree"]
    gather = packed or fused
    if gather:   # the tree's buffers, once, before any step
        md.medusa_build_tree(x["choices"], o["heads"]["topk_ids"].zero_(), x["root"], x["plen"],
                             p_max=t["retrieve"].shape[0], out=t)
        torch.cuda.synchronize()
        assert t["status"].tolist() == [0, -1]
    _reset(x, o, gather)
    torch.cuda.synchronize()
    _step(x, o, k, d, packed, fused)
    torch.cuda.synchronize()
    ref = {n: v.clone() for n, v in _outputs(o, gather).items()}
    if not gather:
        assert int(ref["tree.status"][0]) == 0

    graph = torch.cuda.CUDAGraph()
    _reset(x, o, gather)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _step(x, o, k, d, packed, fused)
    torch.cuda.synchronize()

    for rep in range(4):
        _reset(x, o, gather)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, v in _outputs(o, gather).items():
            assert torch.equal(v, ref[n]), "replay %d: %s differs from the eager step" % (rep, n)
