"""Parity cases: seeded inputs, oracle expectations, comparisons.

The inputs come from ``synth``; the expected values from ``oracle`` only.
Where a float decides an integer (top-k order, an acceptance test), the
cases redraw inputs until the oracle's decision margins exceed float error,
recording the retry counts.
"""

import numpy as np
import torch

import oracle
import synth


# ------------------------------------------------------------------ compare
def rel_err(got, ref):
    """max |g - o| / max(|o|, rms(o)) over all elements (rms floor for
    near-zero references)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    o = np.asarray(ref, dtype=np.float64).ravel()
    if o.size == 0:
        return 0.0
    floor = max(float(np.sqrt(np.mean(o * o))), 1e-30)
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), floor)))


def tol(dtype):
    """Float tolerance: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs."""
    return 1e-4 if dtype == "f32" else 2e-2


def to_dev(a, dtype=None, device="cuda"):
    """NumPy array -> torch device tensor (uint16 arrays are bf16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def to_host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ------------------------------------------------------------------ heads
def heads_case(w, seed=0, margin=1e-3, max_retries=40):
    """Inputs and oracle results for the heads; each head's lm_head is
    redrawn until the gaps between its top-(k+1) fp64 logits are >= margin
    for every sequence."""
    K, k = w["K"], w["topk"]
    retries = [0] * K
    x = synth.heads_inputs(w, seed=seed, retries=retries)
    for _ in range(max_retries):
        r = oracle.resblock(x["hidden"], x["w1"], x["b1"])
        bad = []
        ref_ids = np.empty((w["B"], K, k), dtype=np.int32)
        ref_vals = np.empty((w["B"], K, k))
        for j in range(K):
            z = oracle.lm_head_logits(r, x["w_lm"], head=j)
            ids, vals = oracle.topk_by_value(z, min(k + 1, w["V"]))
            ref_ids[:, j] = ids[:, :k]
            ref_vals[:, j] = vals[:, :k]
            if np.any(np.diff(-vals, axis=1) < margin):
                bad.append(j)
        if not bad:
            return dict(inputs=x, r=r, topk_ids=ref_ids, topk_logits=ref_vals, retries=retries)
        for j in bad:
            retries[j] += 1
        x = synth.heads_inputs(w, seed=seed, retries=retries)
    raise RuntimeError("no margin after %d redraws" % max_retries)


# ------------------------------------------------------------------ tree
def tree_spec(w, seed=0):
    if w["tree"] == "full":
        return synth.full_tree_choices(w["K"], w["topk"])
    return synth.random_tree_choices(w["depth_counts"], w["topk"], seed=seed, workload_id=w["wid"])


def tree_case(w, seed=0, choices=None):
    choices = tree_spec(w, seed) if choices is None else choices
    ch = synth.choices_array(choices, w["K"])
    ids = synth.topk_ids_input(w, seed=seed)
    root = synth.root_token_input(w, seed=seed)
    plen = synth.prefix_lengths(w, seed=seed)
    ref = oracle.build_tree(ch, w["K"], w["topk"], ids, root, plen)
    return dict(choices=ch, topk_ids=ids, root=root, prefix_len=plen, ref=ref)


# ------------------------------------------------------------------ posterior
def posterior_margins_ok(logits, ref_tree, temperature, eps, delta, rel=1e-3):
    """Decisions far from float error: for every node, the argmax beats the
    runner-up by >= rel (relative to 1) and, in typical mode, every child's
    p differs from its parent's threshold by >= rel * threshold."""
    cand = ref_tree["tree_candidates"]
    parent = ref_tree["parent"]
    B, T, V = logits.shape
    for b in range(B):
        st = oracle.node_statistics(logits[b], temperature)
        x = logits[b].astype(np.float64)
        top2 = -np.sort(-x, axis=1)[:, :2]
        if np.any(top2[:, 0] - top2[:, 1] < rel):
            return False
        if temperature > 0:
            thr = np.minimum(np.float32(eps), np.float32(delta) * np.exp(-st["H"]))
            for c in range(1, T):
                n = parent[c]
                p = np.exp(st["z"][n, cand[b, c]] - st["m"][n]) / st["S"][n]
                if abs(p - thr[n]) < rel * thr[n]:
                    return False
    return True


def non_planted_children_clear(logits, ref_tree, plan):
    """No row outside the planted path has one of its children as argmax."""
    cand, parent = ref_tree["tree_candidates"], ref_tree["parent"]
    B, T, _ = logits.shape
    for b in range(B):
        planted = set()
        if plan[b] is not None:
            p, A = plan[b]
            planted = {int(ref_tree["retrieve"][p, j]) for j in range(A)}
        am = np.argmax(logits[b], axis=1)
        for c in range(1, T):
            n = int(parent[c])
            if n not in planted and cand[b, c] == am[n]:
                return False
    return True


def posterior_case(w, tcase, temperature, seed=0, max_retries=50):
    ref = tcase["ref"]
    for retry in range(max_retries):
        logits, plan = synth.posterior_logits(w, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                              ref["depth"], seed=seed + 1000 * retry)
        if not non_planted_children_clear(logits, ref, plan):
            continue
        if not posterior_margins_ok(logits, ref, temperature, w["eps"], w["delta"]):
            continue
        exp = oracle.evaluate_posterior(logits, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                        temperature, w["eps"], w["delta"])
        return dict(logits=logits, plan=plan, ref=exp, retry=retry)
    raise RuntimeError("no margin after %d redraws" % max_retries)
