"""GPU parity of medusa_evaluate_posterior_nucleus against the oracle.

Every node's draw, the best path, accepted length and next token equal the
oracle's bit for bit on inputs whose nucleus decisions sit clear of float
ties.  The nucleus boundary and the inverse-CDF crossing compare sums of
thousands of probabilities: exact sums of fp32 exponentials rounded to 40
fraction bits on the GPU, fp64 in the oracle, so they agree to about 1e-6
of the row's mass; inputs are redrawn until every decision clears 1e-5.  Cases:
planted Vicuna-7B logits (64 nodes, V 32000) at top_p 0.8 and 0.95; three
sequences of 15 nodes over a 1000-token vocabulary (partial thread chunks);
top_p 1 (the whole vocabulary); a tiny top_p, where the draw is the argmax
and the result equals greedy acceptance; equal logits and a tie group at
the nucleus boundary spread over many threads' chunks (ties go to the
lower ids); rows whose boundary bucket holds hundreds to tens of thousands
of tokens (each selection path of the kernel); a one-token vocabulary; a
40000-token vocabulary, past the LDS-resident limit (the segmented kernel).
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import nucleus_case, nucleus_margins, to_dev, to_host, tree_case

pytestmark = pytest.mark.gpu


def _gpu(logits, cand, retrieve, num_paths, temperature, top_p, u):
    out = md.medusa_evaluate_posterior_nucleus(to_dev(logits), to_dev(cand), to_dev(retrieve),
                                               to_dev(np.array([num_paths], dtype=np.int32)), temperature, top_p,
                                               to_dev(np.asarray(u, dtype=np.float32)), keep_samples=True)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _compare(got, ref):
    assert got["samples"].tolist() == ref["samples"].tolist()
    assert got["best_path"].tolist() == ref["best_path"].tolist()
    assert got["accept_len"].tolist() == ref["accept_len"].tolist()
    assert got["next_token"].tolist() == ref["next_token"].tolist()


@pytest.mark.parametrize("top_p", [0.8, 0.95])
@pytest.mark.parametrize("seed", range(2))
def test_nucleus_vicuna7b_planted(gpu_device, seed, top_p):
    w = synth.workload("vicuna-7b")
    tc = tree_case(w, seed=seed)
    nc = nucleus_case(w, tc, 0.7, top_p, seed=seed)
    t = tc["ref"]
    print("seed", seed, "top_p", top_p, "retry", nc["retry"], "plan", nc["plan"], "accept",
          nc["ref"]["accept_len"], flush=True)
    got = _gpu(nc["logits"], t["tree_candidates"], t["retrieve"], t["num_paths"], 0.7, top_p, nc["uniforms"])
    _compare(got, nc["ref"])
    # a planted child dominates its parent's distribution: its nucleus is the
    # child alone, so the planted steps are always accepted
    assert int(nc["ref"]["accept_len"][0]) >= nc["plan"][0][1]


def test_nucleus_batch_ragged_vocab(gpu_device):
    w = synth.workload("tiny-f32", B=3, V=1000, logit_std=2.0, planted=True)
    tc = tree_case(w, seed=2)
    nc = nucleus_case(w, tc, 0.9, 0.8, seed=2)
    t = tc["ref"]
    got = _gpu(nc["logits"], t["tree_candidates"], t["retrieve"], t["num_paths"], 0.9, 0.8, nc["uniforms"])
    _compare(got, nc["ref"])


def test_nucleus_whole_vocabulary(gpu_device):
    w = synth.workload("tiny-f32", B=2, V=777, logit_std=1.0, planted=False)
    tc = tree_case(w, seed=4)
    nc = nucleus_case(w, tc, 1.0, 1.0, seed=4)
    t = tc["ref"]
    got = _gpu(nc["logits"], t["tree_candidates"], t["retrieve"], t["num_paths"], 1.0, 1.0, nc["uniforms"])
    _compare(got, nc["ref"])


def test_nucleus_tiny_top_p_is_greedy(gpu_device):
    w = synth.workload("vicuna-7b", B=2, V=5000)
    tc = tree_case(w, seed=5)
    t = tc["ref"]
    logits, _ = synth.posterior_logits(w, t["tree_candidates"], t["retrieve"], t["num_paths"], t["depth"], seed=5)
    u = synth.node_uniforms(w, logits.shape[1], seed=5)
    got = _gpu(logits, t["tree_candidates"], t["retrieve"], t["num_paths"], 0.7, 1e-7, u)
    assert got["samples"].tolist() == np.argmax(logits, axis=2).tolist()
    greedy = md.medusa_evaluate_posterior(to_dev(logits), to_dev(t["tree_candidates"]), to_dev(t["retrieve"]),
                                          to_dev(np.array([t["num_paths"]], dtype=np.int32)), 0.0, 0.09, 0.3)
    torch.cuda.synchronize()
    for key in ("best_path", "accept_len", "next_token"):
        assert got[key].tolist() == to_host(greedy[key]).tolist()
    ref = oracle.evaluate_posterior(logits, t["tree_candidates"], t["retrieve"], t["num_paths"], 0.0, 0.09, 0.3)
    assert got["accept_len"].tolist() == ref["accept_len"].tolist()


def _star(rows, children, temperature, top_p, u):
    """Root with the given logit rows (one per node) and children tokens."""
    T = rows.shape[0]
    cand = np.array([[0] + list(children)], dtype=np.int32)
    retrieve = np.array([[0, 1 + c] for c in range(len(children))], dtype=np.int32)
    logits = rows[None].astype(np.float32)
    ref = oracle.evaluate_posterior_nucleus(logits, cand, retrieve, len(children), temperature, top_p,
                                            np.asarray(u, dtype=np.float32)[None])
    got = _gpu(logits, cand, retrieve, len(children), temperature, top_p, np.asarray(u, dtype=np.float32)[None])
    assert T == 1 + len(children)
    return got, ref


def test_nucleus_equal_logits(gpu_device):
    # 1000 equal tokens, top_p 0.4555: the nucleus is ids 0..455 (456
    # tokens); the draw is id floor(u * 456) for u clear of the grid
    V, n = 1000, 456
    us = [0.0, 0.1, 0.501, 0.73, 0.999]
    rows = np.zeros((len(us), V), dtype=np.float32)
    got, ref = _star(rows, [3, 200, 455, 456], 1.0, 0.4555, us)
    assert ref["samples"][0].tolist() == [int(x * n) for x in us]
    _compare(got, ref)


def test_nucleus_tie_group_at_the_boundary(gpu_device):
    # three tokens at logit 2 and ten at logit 0 spread over four 256-token
    # tiles, the rest far below: top_p puts the boundary inside the group of
    # ten, so its lowest ids complete the nucleus
    V = 1100
    row = np.full(V, -60.0, dtype=np.float32)
    hi = [40, 700, 1099]
    group = [5, 90, 255, 256, 300, 511, 512, 800, 1000, 1098]
    row[hi] = 2.0
    row[group] = 0.0
    e2 = np.exp(2.0)
    Z = 3 * e2 + 10
    # mass of the three + 4.5 group tokens (boundary mid-token: 5 taken)
    top_p = (3 * e2 + 4.5) / Z
    ids, _ = oracle.nucleus(row, 1.0, top_p)
    assert ids.tolist() == sorted(hi + group[:5])
    # the nucleus in id order: 5 (1), 40 (e^2), 90, 255, 256, 300 (1 each),
    # 700, 1099 (e^2 each); one uniform at the middle of each token's share
    # of the CDF, plus u = 0
    mass = np.array([1, e2, 1, 1, 1, 1, e2, e2])
    cdf = np.cumsum(mass) / mass.sum()
    us = np.concatenate([[0.0], cdf - mass / mass.sum() / 2])
    for u in us[1:]:
        assert nucleus_margins(row, 1.0, top_p, u) > 1e-2
    rows = np.tile(row, (len(us), 1))
    children = [group[0], hi[1], group[6], 2, group[4], group[5], hi[2], 40]
    got, ref = _star(rows, children, 1.0, top_p, us)
    assert ref["samples"][0].tolist() == [5, 5, 40, 90, 255, 256, 300, 700, 1099]
    _compare(got, ref)


def _crowded_rows(V, cluster, seed):
    """Rows whose first selection bucket (linear in value over the row's
    range) holds many tokens: one far outlier below stretches the range, so
    a cluster of `cluster` tokens with distinct values inside a 0.01-wide
    interval falls into one bucket; the rest sit 12 below the cluster."""
    rng = np.random.default_rng(seed)
    row = np.full(V, -12.0, dtype=np.float32) + rng.uniform(0, 1e-3, V).astype(np.float32)
    ids = rng.choice(np.arange(1, V), size=cluster, replace=False)
    row[ids] = (1.0 + rng.uniform(0, 1e-2, cluster)).astype(np.float32)
    row[0] = -60.0
    return row


@pytest.mark.parametrize("V,cluster", [(32000, 2000), (32000, 20000), (4000, 600)])
def test_nucleus_crowded_boundary_bucket(gpu_device, V, cluster):
    # the boundary bucket then holds more tokens than the direct resolution
    # takes: at most 4096 of them are gathered into a list for the radix
    # passes, a larger bucket is walked over the whole row
    temperature, top_p = 0.7, 0.8
    rows, us = [], []
    for r in range(3):
        for attempt in range(20):
            row = _crowded_rows(V, cluster, seed=100 * r + attempt)
            u = float(np.float32((r + 0.37) / 3.0))
            if nucleus_margins(row, temperature, top_p, u) > 1e-5:
                break
        else:
            pytest.fail("no row cleared the margins")
        rows.append(row)
        us.append(u)
    rows = np.stack(rows)
    children = [int(np.argmax(rows[0])), 7]
    got, ref = _star(rows, children, temperature, top_p, us)
    _compare(got, ref)


def test_nucleus_one_token_vocabulary(gpu_device):
    rows = np.zeros((3, 1), dtype=np.float32)
    got, ref = _star(rows, [0, 0], 0.5, 0.8, [0.2, 0.9, 0.5])
    assert got["samples"].tolist() == [[0, 0, 0]]
    _compare(got, ref)
    assert got["accept_len"].tolist() == [1]


def test_nucleus_long_vocabulary(gpu_device):
    # rows longer than the LDS-resident limit (32768 tokens) take the
    # segmented kernel: two segments of 32768, the second ragged
    w = synth.workload("tiny-f32", B=1, V=40000, logit_std=3.0, planted=True)
    tc = tree_case(w, seed=6)
    nc = nucleus_case(w, tc, 0.7, 0.8, seed=6)
    t = tc["ref"]
    got = _gpu(nc["logits"], t["tree_candidates"], t["retrieve"], t["num_paths"], 0.7, 0.8, nc["uniforms"])
    _compare(got, nc["ref"])
