"""Nucleus (top-p) acceptance of the candidate tree -- TEST INFRASTRUCTURE ONLY.

Definition followed: API reference page, the signatures of
``medusa_generate``, ``generate_candidates`` and ``evaluate_posterior``,
which carry a ``top_p`` argument (default 0.8) beside the ``sampling`` mode
(default typical).  The pages name the parameter and nothing more; the
reading taken here is the plainest one consistent with the rest of the
method (a candidate is kept when it agrees with what the base model would
have produced at its parent, and the step yields the base model's own next
token):

  * p_n = softmax(logits_n / temperature) at node n (temperature > 0).
  * The nucleus of node n: order the vocabulary by p_n descending, ties by
    token id ascending; the nucleus is the shortest prefix of that order
    whose probability mass reaches top_p.
  * One token s_n is drawn from the nucleus renormalised, by inverse CDF
    with a caller-supplied uniform u_n in [0, 1), walking the nucleus in
    token-id order: s_n is the first token whose running mass exceeds
    u_n * (nucleus mass).  (If rounding leaves no such token, the nucleus's
    highest id.)
  * A child c of parent n is accepted exactly when its token equals s_n.
    The best path is the lowest-index path of maximal accepted length, and
    the next token is s at the last accepted node.

With these rules a step emits tokens distributed exactly as nucleus sampling
of the base model would (each accepted token is the sample itself).  fp64
throughout from the float32 inputs; temperature, top_p and u are taken at
float32 precision, as float32 arguments hold them.
"""

import numpy as np

from .common import as_f64


def _f32(x):
    return float(np.float32(x))


def nucleus(logits_row, temperature, top_p):
    """The nucleus of one node: (token ids ascending, their probabilities).

    Probabilities are p_n (not renormalised over the nucleus).
    """
    t, q = _f32(temperature), _f32(top_p)
    if not t > 0.0:
        raise ValueError("temperature must be positive")
    if not 0.0 < q <= 1.0:
        raise ValueError("top_p must lie in (0, 1]")
    z = as_f64(logits_row) / t
    p = np.exp(z - z.max())
    p /= p.sum()
    V = p.shape[0]
    order = np.lexsort((np.arange(V), -p))      # p descending, then id ascending
    mass = np.cumsum(p[order])
    k = min(int(np.searchsorted(mass, q, side="left")), V - 1)   # first prefix reaching top_p
    ids = np.sort(order[:k + 1])
    return ids, p[ids]


def nucleus_sample(logits_row, temperature, top_p, u):
    """The token drawn from one node's nucleus with uniform u."""
    ids, p = nucleus(logits_row, temperature, top_p)
    target = min(max(_f32(u), 0.0), 1.0) * p.sum()
    run = 0.0
    for v, pv in zip(ids, p):
        run += pv
        if run > target:
            return int(v)
    return int(ids[-1])


def evaluate_posterior_nucleus(logits, tree_candidates, retrieve, num_paths, temperature, top_p, uniforms):
    """Best path, accepted length, next token and every node's sample.

    logits [B][T][V] float32, tree_candidates [B][T], retrieve [P][D]
    (-1 padded), num_paths, uniforms [B][T] in [0, 1).
    Returns dict with best_path, accept_len, next_token ([B]), samples
    [B][T] and path_len [B][P].
    """
    logits = np.asarray(logits)
    B, T, _ = logits.shape
    ret = np.asarray(retrieve)
    u = np.asarray(uniforms, dtype=np.float32)
    P = int(num_paths)
    D = ret.shape[1]
    samples = np.zeros((B, T), dtype=np.int64)
    best = np.zeros(B, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    path_len = np.zeros((B, P), dtype=np.int64)
    for b in range(B):
        for n in range(T):
            samples[b, n] = nucleus_sample(logits[b, n], temperature, top_p, u[b, n])
        for p in range(P):
            ell = 0
            for j in range(1, D):
                c = int(ret[p, j])
                if c < 0 or c >= T:
                    break
                if int(tree_candidates[b][c]) != samples[b, int(ret[p, j - 1])]:
                    break
                ell += 1
            path_len[b, p] = ell
        bp = int(np.argmax(path_len[b])) if P > 0 else 0
        best[b] = bp
        acc[b] = path_len[b, bp] if P > 0 else 0
        last = int(ret[bp, acc[b]]) if P > 0 else 0
        nxt[b] = samples[b, last]
    return dict(best_path=best, accept_len=acc, next_token=nxt, samples=samples, path_len=path_len)
