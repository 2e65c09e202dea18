"""GPU parity of the base model forward pieces and of greedy generation.

The pieces (embedding rows, residual add + RMSNorm, RoPE with the KV-cache
scatter, SiLU-gate x up) match the oracle's definitions to one bf16
rounding.  A whole forward of a tiny LLaMA-style model (H 256, 4 heads x 64,
MLP 512, 2 layers) over prompts of 1, 20 and 200 tokens gives the oracle's
logits within max relative error 2e-2, each element against
max(|o|, rms(o)) (bf16 activations at the norms, attention and MLP).  A candidate tree run through the model after a prefix
gives, at every node, the logits of the prefix followed by that node's path
(the oracle recomputes each path as a plain sequence).  Plain greedy
decoding on the GPU emits the oracle's greedy continuation; Medusa greedy
decoding emits exactly the same tokens, with random heads and with heads
fitted to the continuation (which accept long paths, through second-ranked
branches too).
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import fitted_heads, rel_err, to_dev, to_host
from speculative_decoding_medusa_amd.decoder import TinyDecoder

pytestmark = pytest.mark.gpu

CFG = dict(H=256, heads=4, I=512, layers=2, V=1000, eps=1e-6, theta=10000.0)


def _rel(got, ref):
    # max |g - o| / max(|o|, rms(o)), the float bar for bf16 work
    return rel_err(got, ref)


def _bf16_to_f64(t):
    return oracle.as_f64(to_host(t.view(torch.int16)).view(np.uint16))


def test_embed_and_rmsnorm(gpu_device):
    m = synth.tiny_decoder(CFG, seed=1)
    toks = np.array([[3, 999, 0, 500, 3]], dtype=np.int32)
    x = md.medusa_embed(to_dev(toks), to_dev(m["embed"]))
    torch.cuda.synchronize()
    E = oracle.as_f64(m["embed"])
    assert np.array_equal(to_host(x)[0], E[toks[0]].astype(np.float32))
    # residual add + norm: x += y, out = rmsnorm(x) * g in bf16
    y = np.random.default_rng(0).standard_normal((1, 5, CFG["H"])).astype(np.float32)
    x0 = to_host(x).astype(np.float64)
    out = md.medusa_add_rmsnorm(x, to_dev(m["final_norm"]), 1e-6, y=to_dev(y))
    torch.cuda.synchronize()
    ref = oracle.decoder.rmsnorm(x0 + y, m["final_norm"], 1e-6)
    assert np.allclose(to_host(x), (x0 + y).astype(np.float32), rtol=1e-6, atol=1e-6)
    assert _rel(_bf16_to_f64(out), ref) < 8e-3
    out2 = md.medusa_add_rmsnorm(x, to_dev(m["final_norm"]), 1e-6)    # no add
    torch.cuda.synchronize()
    assert _rel(_bf16_to_f64(out2), ref) < 8e-3


def test_rope_qkv_and_cache_slots(gpu_device):
    B, T, heads, d, S = 2, 7, 4, 64, 40
    rng = np.random.default_rng(2)
    qkv = rng.standard_normal((B, T, 3, heads, d)).astype(np.float32)
    pos = np.array([[5, 6, 6, 7, 7, 8, 9], [0, 1, 2, 3, 4, 5, 6]], dtype=np.int32)
    plen = np.array([5, 30], dtype=np.int32)
    kc = torch.full((B, heads, S, d), 7.0, dtype=torch.bfloat16, device=gpu_device)
    vc = torch.full((B, heads, S, d), 7.0, dtype=torch.bfloat16, device=gpu_device)
    q = md.medusa_rope_qkv(to_dev(qkv), to_dev(pos), to_dev(plen), 10000.0, kc, vc)
    torch.cuda.synchronize()
    kh, vh = _bf16_to_f64(kc), _bf16_to_f64(vc)
    for b in range(B):
        rq = oracle.decoder.rope(qkv[b, :, 0], pos[b], 10000.0)
        rk = oracle.decoder.rope(qkv[b, :, 1], pos[b], 10000.0)
        assert _rel(_bf16_to_f64(q)[b], rq) < 8e-3
        sl = slice(plen[b], min(plen[b] + T, S))
        n = sl.stop - sl.start
        assert _rel(kh[b][:, sl].transpose(1, 0, 2), rk[:n]) < 8e-3
        assert _rel(vh[b][:, sl].transpose(1, 0, 2), qkv[b, :n, 2]) < 8e-3
        keep = np.ones(S, dtype=bool)
        keep[sl] = False
        assert np.all(kh[b][:, keep] == 7.0) and np.all(vh[b][:, keep] == 7.0)


def test_silu_mul(gpu_device):
    rng = np.random.default_rng(3)
    gu = (rng.standard_normal((9, 2 * 48)) * 3).astype(np.float32)
    out = md.medusa_silu_mul(to_dev(gu))
    torch.cuda.synchronize()
    g, u = gu[:, :48].astype(np.float64), gu[:, 48:].astype(np.float64)
    assert _rel(_bf16_to_f64(out), oracle.decoder.silu(g) * u) < 8e-3


@pytest.mark.parametrize("P", [1, 20, 200])
def test_prefill_logits_match_oracle(gpu_device, P):
    m = synth.tiny_decoder(CFG, seed=1)
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    prompt = [int(t) for t in np.random.default_rng(P).integers(CFG["V"], size=P)]
    _, lg = dec.prefill(prompt)
    torch.cuda.synchronize()
    ref, _ = oracle.decoder.forward(m, prompt)
    assert _rel(to_host(lg)[0], ref) < 2e-2


def test_tree_forward_matches_path_sequences(gpu_device):
    m = synth.tiny_decoder(CFG, seed=4)
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    rng = np.random.default_rng(4)
    prompt = [int(t) for t in rng.integers(CFG["V"], size=30)]
    dec.prefill(prompt)
    K, k = 3, 3
    choices = synth.choices_array(synth.random_tree_choices([3, 5, 4], k, seed=4), K)
    ids = rng.integers(CFG["V"], size=(1, K, k)).astype(np.int32)
    plen = to_dev(np.array([30], dtype=np.int32))
    tree = md.medusa_build_tree(to_dev(choices), to_dev(ids), to_dev(np.array([17], dtype=np.int32)), plen)
    _, lg = dec.forward(tree["tree_candidates"], tree["position_ids"], plen, tree["tree_mask"])
    torch.cuda.synchronize()
    cand = to_host(tree["tree_candidates"])[0]
    parent = to_host(tree["parent"])
    got = to_host(lg)[0]
    for node in range(len(cand)):
        path, p = [], node
        while p >= 0:
            path.append(int(cand[p]))
            p = int(parent[p]) if p > 0 else -1
        ref, _ = oracle.decoder.forward(m, prompt + path[::-1])
        assert _rel(got[node], ref[-1]) < 2e-2, node


def _prompt_with_margin(model, P, n, min_gap, seeds):
    """A prompt whose greedy continuation keeps every top-2 logit gap above
    min_gap (far above the GPU's logit error)."""
    for s in seeds:
        prompt = [int(t) for t in np.random.default_rng(s).integers(model["cfg"]["V"], size=P)]
        toks, gaps = oracle.decoder.greedy_decode(model, prompt, n)
        if min(gaps) >= min_gap:
            return prompt, toks
    raise RuntimeError("no prompt with margin")


@pytest.mark.parametrize("V", [64, 1000])
def test_greedy_and_medusa_match_oracle(gpu_device, V):
    cfg = dict(CFG, V=V)
    m = synth.tiny_decoder(cfg, seed=1)
    n = 32
    prompt, ref = _prompt_with_margin(m, 12, n, 0.06, range(40))
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    assert dec.greedy(prompt, n) == ref
    K, topk = 3, 8
    hd = synth.tiny_heads(cfg, K, seed=2)
    heads = {key: to_dev(v) for key, v in hd.items()}
    choices = to_dev(synth.choices_array(synth.random_tree_choices([6, 8, 6], topk, seed=3), K))
    toks, accepts, _ = TinyDecoder(m, gpu_device, max_slots=256).medusa(heads, choices, topk, prompt, n)
    print("V", V, "accepts", accepts, flush=True)
    assert toks == ref


def test_medusa_with_fitted_heads(gpu_device):
    cfg = dict(CFG, V=1000)
    m = synth.tiny_decoder(cfg, seed=1)
    n, K = 40, 3
    prompt, ref = _prompt_with_margin(m, 12, n, 0.06, range(40))
    hd, cont = fitted_heads(m, prompt, n, K, seed=5)
    assert cont == ref
    heads = {key: to_dev(v) for key, v in hd.items()}
    # full binary tree of depth 3: rank-0 and rank-1 branches everywhere
    choices = to_dev(synth.choices_array(synth.full_tree_choices(K, 2), K))
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    toks, accepts, paths = dec.medusa(heads, choices, 2, prompt, n)
    print("accepts", accepts, "best paths", paths, flush=True)
    assert toks == ref
    assert np.mean(accepts) >= 2.0
    assert len(accepts) <= n // 2
    assert any(p != 0 for p in paths)   # second-ranked branches accepted too


def test_generation_replayed_from_hip_graphs(gpu_device):
    # the same loops with each step captured once and replayed: every
    # replayed step's token lands in the device-side output buffer, and the
    # sequences equal the eager ones (and the oracle's)
    cfg = dict(CFG, V=1000)
    m = synth.tiny_decoder(cfg, seed=1)
    n, K = 40, 3
    prompt, ref = _prompt_with_margin(m, 12, n, 0.06, range(40))
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    assert dec.greedy_graph(prompt, n) == ref
    hd, _ = fitted_heads(m, prompt, n, K, seed=5)
    heads = {key: to_dev(v) for key, v in hd.items()}
    choices = to_dev(synth.choices_array(synth.full_tree_choices(K, 2), K))
    eager, accepts, _ = dec.medusa(heads, choices, 2, prompt, n)
    toks, steps = dec.medusa_graph(heads, choices, 2, prompt, n, check_every=3)
    assert eager == ref and toks == ref
    assert steps >= len(accepts)    # may overshoot by up to check_every steps
    # random heads: one token per step, still the same sequence
    rnd = {key: to_dev(v) for key, v in synth.tiny_heads(cfg, K, seed=2).items()}
    toks, steps = dec.medusa_graph(rnd, choices, 2, prompt, n)
    assert toks == ref


def _tree_parents(choices, K, topk):
    # the tree's parent array depends only on the spec
    return oracle.build_tree(choices, K, topk, np.zeros((1, K, topk), dtype=np.int32), np.zeros(1, np.int32),
                             np.zeros(1, np.int32))["parent"]


@pytest.mark.parametrize("mode", ["typical", "nucleus"])
def test_sampled_medusa_decisions_match_oracle(gpu_device, mode):
    # Medusa decoding in a sampled mode; every step's decisions -- best path,
    # accepted length, the drawn next root, and the prompt's first root --
    # equal the oracle's on the step's own logits (the base forward is
    # checked against the oracle's on its own elsewhere) with the same
    # Philox keys, wherever the decision clears float error
    from cases import nucleus_margins, posterior_margins_ok, typical_sample_robust
    from oracle import sampling as smp
    cfg = dict(CFG, V=1000)
    m = synth.tiny_decoder(cfg, seed=1)
    n, K, k = 40, 3, 2
    prompt, _ = _prompt_with_margin(m, 12, n, 0.06, range(40))
    hd, _ = fitted_heads(m, prompt, n, K, seed=5)
    heads = {key: to_dev(v) for key, v in hd.items()}
    choices = synth.choices_array(synth.full_tree_choices(K, k), K)
    parent = _tree_parents(choices, K, k)
    t, eps, delta, top_p, seed = 0.7, 0.09, 0.3, 0.8, 21
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    rec = []
    toks, accepts = dec.medusa_sampled(heads, to_dev(choices), k, prompt, n, mode=mode, temperature=t, eps=eps,
                                       delta=delta, top_p=top_p, seed=seed, record=rec)
    print("mode", mode, "accepts", accepts, flush=True)
    checked = 0
    r0 = rec[0]
    row0 = r0["logits"][0, 0]
    if mode == "typical":
        u = smp.uniform(seed, 0, 0, 0, smp.PURPOSE_NEXT_TOKEN)
        if typical_sample_robust(row0, t, eps, delta, u):
            assert r0["next_token"] == smp.typical_sample(row0, t, eps, delta, u)
            checked += 1
    else:
        u = smp.uniform(seed, 0, 0, 0, smp.PURPOSE_NUCLEUS)
        if nucleus_margins(row0, t, top_p, u) >= 1e-5:
            assert r0["next_token"] == oracle.nucleus_sample(row0, t, top_p, u)
            checked += 1
    emitted = []
    root = r0["next_token"]
    for r in rec[1:]:
        s, lg, cand, ret, P = r["step"], r["logits"], r["tree_candidates"], r["retrieve"], r["num_paths"]
        assert int(cand[0, 0]) == root
        T = cand.shape[1]
        if mode == "typical":
            ok = posterior_margins_ok(lg, dict(tree_candidates=cand, parent=parent), t, eps, delta)
            if ok:
                exp = oracle.evaluate_posterior(lg, cand, ret, P, t, eps, delta)
                assert (r["best_path"], r["accept_len"]) == (int(exp["best_path"][0]), int(exp["accept_len"][0]))
                node = int(ret[r["best_path"], r["accept_len"]])
                u = smp.uniform(seed, s, 0, 0, smp.PURPOSE_NEXT_TOKEN)
                if typical_sample_robust(lg[0, node], t, eps, delta, u):
                    assert r["next_token"] == smp.typical_sample(lg[0, node], t, eps, delta, u)
                    checked += 1
        else:
            u = smp.uniforms(seed, s, 1, T, smp.PURPOSE_NUCLEUS)
            if all(nucleus_margins(lg[0, j], t, top_p, u[0, j]) >= 1e-5 for j in range(T)):
                exp = oracle.evaluate_posterior_nucleus(lg, cand, ret, P, t, top_p, u)
                assert (r["best_path"], r["accept_len"], r["next_token"]) == (
                    int(exp["best_path"][0]), int(exp["accept_len"][0]), int(exp["next_token"][0]))
                checked += 1
        path = ret[r["best_path"]]
        emitted.extend(int(cand[0, path[j]]) for j in range(r["accept_len"] + 1))
        root = r["next_token"]
    assert emitted[:n] == toks
    assert checked >= 0.8 * len(rec), (checked, len(rec))


def test_sampling_at_low_temperature_is_greedy(gpu_device):
    # as the temperature goes to 0 the typical set shrinks to the argmax:
    # plain and Medusa sampled decoding then emit the greedy tokens
    cfg = dict(CFG, V=1000)
    m = synth.tiny_decoder(cfg, seed=1)
    n, K = 24, 3
    prompt, ref = _prompt_with_margin(m, 12, n, 0.06, range(40))
    dec = TinyDecoder(m, gpu_device, max_slots=256)
    assert dec.sample(prompt, n, mode="typical", temperature=1e-3, seed=4) == ref
    hd, _ = fitted_heads(m, prompt, n, K, seed=5)
    heads = {key: to_dev(v) for key, v in hd.items()}
    choices = to_dev(synth.choices_array(synth.full_tree_choices(K, 2), K))
    toks, accepts = TinyDecoder(m, gpu_device, max_slots=256).medusa_sampled(heads, choices, 2, prompt, n,
                                                                             mode="typical", temperature=1e-3,
                                                                             seed=4)
    assert toks == ref and np.mean(accepts) >= 1.5
