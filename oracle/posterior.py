"""Acceptance of the candidate tree (test infrastructure only).

Definition followed:
  * API reference page, ``evaluate_posterior`` (arguments ``temperature``,
    ``posterior_threshold``, ``posterior_alpha``) and ``medusa_generate``
    (defaults temperature 0.0, posterior_threshold 0.09,
    posterior_alpha 0.3).
  * Study notes, 核心要点 (typical acceptance: keep a candidate whose base
    probability is typical enough instead of rejection sampling) and 实践案例
    案例 1 (keep the longest acceptable prefix walking from the root towards
    a leaf); 学到什么 (each verify step also yields the base model's own next
    token).

Readings where the pages are silent: temperature 0 means greedy, accepting a
candidate exactly when it equals the base argmax at its parent; otherwise a
candidate x at parent n is accepted when p_n(x) > min(eps, delta *
exp(-H(p_n))), with p_n = softmax(logits_n / temperature) and H the natural-
log entropy; eps = posterior_threshold and delta = posterior_alpha.  The
best path is the lowest-index path of maximal accepted length; the next
token is the base argmax at the last accepted node (in both modes).
"""

import numpy as np

from .common import as_f64


def _f32(x):
    return float(np.float32(x))


def node_statistics(logits_row_block, temperature):
    """Per-node quantities of the base distribution.

    logits [T][V] (float32 values).  Returns dict with argmax [T] (first
    maximum) and, when temperature > 0, m [T] = max z, S [T] = sum exp(z - m),
    H [T] = -sum p ln p with z = logits / temperature.
    """
    x = as_f64(logits_row_block)
    out = dict(argmax=np.argmax(x, axis=1).astype(np.int64))
    t = _f32(temperature)
    if t > 0.0:
        z = x / t
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        S = e.sum(axis=1)
        A = ((z - m[:, None]) * e).sum(axis=1)
        out.update(z=z, m=m, S=S, H=np.log(S) - A / S)
    return out


def evaluate_posterior(logits, tree_candidates, retrieve, num_paths, temperature, eps, delta):
    """Best path, accepted length and next token per sequence.

    logits [B][T][V] float32 base logits at every tree node,
    tree_candidates [B][T], retrieve [P][D] (-1 padded), num_paths.
    temperature, eps and delta are taken at float32 precision, as a
    float32 argument would hold them.  The greedy test compares token ids;
    the typical test compares p and the threshold after rounding each to
    float32.

    Returns dict with best_path, accept_len, next_token (int arrays [B]),
    path_len [B][P] and the per-node statistics.
    """
    logits = np.asarray(logits)
    B, T, _ = logits.shape
    ret = np.asarray(retrieve)
    P = int(num_paths)
    D = ret.shape[1]
    t, e_, d_ = _f32(temperature), _f32(eps), _f32(delta)
    best = np.zeros(B, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    path_len = np.zeros((B, P), dtype=np.int64)
    stats = []
    for b in range(B):
        st = node_statistics(logits[b], t)
        if t > 0.0:
            thr = np.minimum(e_, d_ * np.exp(-st["H"]))
            st["thr"] = thr

        def accepted(parent, child):
            tok = int(tree_candidates[b][child])
            if t == 0.0:
                return tok == int(st["argmax"][parent])
            p = np.exp(st["z"][parent, tok] - st["m"][parent]) / st["S"][parent]
            return _f32(p) > _f32(st["thr"][parent])

        for p in range(P):
            ell = 0
            for j in range(1, D):
                c = int(ret[p, j])
                if c < 0 or c >= T:
                    break
                if not accepted(int(ret[p, j - 1]), c):
                    break
                ell += 1
            path_len[b, p] = ell
        bp = int(np.argmax(path_len[b])) if P > 0 else 0   # first maximum = lowest index
        best[b] = bp
        acc[b] = path_len[b, bp] if P > 0 else 0
        last = int(ret[bp, acc[b]]) if P > 0 else 0
        nxt[b] = st["argmax"][last]
        stats.append(st)
    return dict(best_path=best, accept_len=acc, next_token=nxt, path_len=path_len, stats=stats)
