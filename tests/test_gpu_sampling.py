"""GPU parity of the counter-based uniforms and the typical-mode sampled
next token, through the C ABI.

medusa_philox_uniforms equals the oracle's Philox4x64-10 uniforms bit for
bit (seeds and steps past 2^63, every purpose, the largest B x T).
medusa_sample_typical equals the oracle's draw at the last accepted node on
inputs whose draw sits clear of float error (the draw is the same with every
near-threshold token counted in or out, and u times the allowed mass is at
least 1e-5 of it from every running-sum boundary; the step of the key is
advanced until it is): planted Vicuna-7B logits (64 nodes, V 32000) at the
best path the acceptance picks, three sequences over 1000 tokens, rows at
the register kernel's edges (4099, 4100, 32767 and 32768 tokens), 40000
tokens (the streaming kernel), a flat row (token floor(u V)) and a dominant
token.  Nucleus
acceptance run on the library's own uniforms equals the oracle's on the
same keys.
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import nucleus_margins, posterior_case, to_dev, to_host, tree_case, typical_sample_robust
from oracle import sampling as smp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,step,purpose,B,T", [
    (0, 0, 0, 1, 64),
    (2 ** 64 - 1, 12345678901, 1, 16, 256),
    (7, 3, 0, 3, 15),
    (2 ** 40 + 3, 2 ** 63 + 1, 5, 1, 1),
])
def test_philox_uniforms_bit_exact(gpu_device, seed, step, purpose, B, T):
    got = to_host(md.medusa_philox_uniforms(seed, step, purpose, B, T, device=gpu_device))
    torch.cuda.synchronize()
    ref = smp.uniforms(seed, step, B, T, purpose)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _gpu_sample(logits, retrieve, best, acc, t, eps, delta, seed, step):
    out = md.medusa_sample_typical(to_dev(logits), to_dev(np.asarray(retrieve, dtype=np.int32)),
                                   to_dev(np.asarray(best, dtype=np.int32)), to_dev(np.asarray(acc, dtype=np.int32)),
                                   t, eps, delta, seed, step)
    torch.cuda.synchronize()
    return to_host(out).tolist()


def _robust_step(logits, retrieve, best, acc, t, eps, delta, seed, tries=200):
    """The first step whose draws (every sequence) are all robust."""
    for step in range(tries):
        ok = True
        for b in range(logits.shape[0]):
            node = int(retrieve[int(best[b]), int(acc[b])])
            u = smp.uniform(seed, step, b, 0, smp.PURPOSE_NEXT_TOKEN)
            if not typical_sample_robust(logits[b, node], t, eps, delta, u):
                ok = False
                break
        if ok:
            return step
    raise RuntimeError("no robust step")


def _check_tree_case(w, seed, t=0.7):
    tc = tree_case(w, seed=seed)
    pc = posterior_case(w, tc, t, seed=seed)
    tr = tc["ref"]
    exp = pc["ref"]
    step = _robust_step(pc["logits"], tr["retrieve"], exp["best_path"], exp["accept_len"], t, w["eps"], w["delta"],
                        seed)
    ref = smp.sample_next_typical(pc["logits"], tr["retrieve"], exp["best_path"], exp["accept_len"], t, w["eps"],
                                  w["delta"], seed, step)
    got = _gpu_sample(pc["logits"], tr["retrieve"], exp["best_path"], exp["accept_len"], t, w["eps"], w["delta"],
                      seed, step)
    print("step", step, "accept", exp["accept_len"], "draws", got, flush=True)
    assert got == ref.tolist()
    return got


@pytest.mark.parametrize("seed", range(4))
def test_sample_typical_vicuna7b(gpu_device, seed):
    _check_tree_case(synth.workload("vicuna-7b"), seed)


def test_sample_typical_three_sequences_small_vocab(gpu_device):
    _check_tree_case(synth.workload("vicuna-7b", B=3, V=1000, logit_std=2.0), 5)


def test_sample_typical_vocab_40000(gpu_device):
    # past 32768 tokens: the streaming kernel
    _check_tree_case(synth.workload("vicuna-7b", V=40000), 6)


@pytest.mark.parametrize("B,V", [
    (2, 32768),    # the register kernel's largest row, 16-byte loads
    (1, 32767),    # its largest row of element loads (V % 4 != 0)
    (3, 4099),     # one id past a 4096-id chunk, element loads
    (2, 4100),     # ragged second chunk, 16-byte loads
])
def test_sample_typical_register_kernel_edges(gpu_device, B, V):
    _check_tree_case(synth.workload("vicuna-7b", B=B, V=V), V % 97)


def test_sample_typical_flat_and_dominant_rows(gpu_device):
    V = 1000
    one = np.array([[0]], dtype=np.int32)
    zero = np.zeros(1, dtype=np.int32)
    flat = np.zeros((1, 1, V), dtype=np.float32)
    for step in range(6):
        u = float(smp.uniform(3, step, 0, 0, smp.PURPOSE_NEXT_TOKEN))
        got = _gpu_sample(flat, one, zero, zero, 0.7, 0.09, 0.3, 3, step)
        assert got == [int(np.floor(u * V))] == [smp.typical_sample(flat[0, 0], 0.7, 0.09, 0.3, u)]
    dom = np.random.default_rng(0).standard_normal((1, 1, V)).astype(np.float32)
    dom[0, 0, 417] = 80.0
    for step in range(3):
        assert _gpu_sample(dom, one, zero, zero, 1.0, 0.09, 0.3, 11, step) == [417]


def test_nucleus_on_library_uniforms(gpu_device):
    w = synth.workload("vicuna-7b")
    tc = tree_case(w, seed=2)
    tr = tc["ref"]
    T = int(tr["tree_candidates"].shape[1])
    for seed in range(40):
        logits, plan = synth.posterior_logits(w, tr["tree_candidates"], tr["retrieve"], tr["num_paths"], tr["depth"],
                                              seed=100 + seed)
        u = smp.uniforms(seed, 9, 1, T, smp.PURPOSE_NUCLEUS)
        if all(nucleus_margins(logits[0, n], 0.7, 0.8, u[0, n]) >= 1e-5 for n in range(T)):
            break
    else:
        raise RuntimeError("no margin")
    ud = md.medusa_philox_uniforms(seed, 9, md.PURPOSE_NUCLEUS, 1, T, device=gpu_device)
    out = md.medusa_evaluate_posterior_nucleus(to_dev(logits), to_dev(tr["tree_candidates"]), to_dev(tr["retrieve"]),
                                               to_dev(np.array([tr["num_paths"]], dtype=np.int32)), 0.7, 0.8, ud,
                                               keep_samples=True)
    torch.cuda.synchronize()
    ref = oracle.evaluate_posterior_nucleus(logits, tr["tree_candidates"], tr["retrieve"], tr["num_paths"], 0.7, 0.8,
                                            u)
    for key in ("samples", "best_path", "accept_len", "next_token"):
        assert to_host(out[key]).tolist() == ref[key].tolist(), key
