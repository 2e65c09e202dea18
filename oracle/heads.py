"""Medusa heads (test infrastructure only).

Definition followed:
  * API reference page ("Medusa API参考：核心函数与类详解"), section on
    MedusaModelABC: ``medusa_head`` is a set of residual blocks and linear
    layers; MedusaConfig gives ``medusa_num_layers`` = 1.
  * Study notes ("Medusa — 让大模型自己同时猜好几个 token"), sections
    是什么 / 核心要点: K parallel heads read the last hidden state; each is a
    one-layer MLP with a residual back to that hidden state and projects to
    vocabulary logits; head k proposes the token at position t+k+1; the
    top-k tokens of each head feed the candidate tree.

Readings where the pages are silent: the MLP activation is SiLU, each head
owns its lm_head (no bias), weights are stored out x in (row i of W1 makes
output i), and the ResBlock output r is carried in full precision into the
lm_head.
"""

import numpy as np

from .common import as_f64


def resblock(hidden, w1, b1):
    """r[b, j, :] = h[b] + SiLU(W1[j] @ h[b] + b1[j]) for every head j.

    hidden [B][H], w1 [K][H][H] (out x in), b1 [K][H]  ->  r [B][K][H] float64.
    SiLU(u) = u * sigmoid(u) = u / (1 + exp(-u)).
    """
    h = as_f64(hidden)
    W1 = as_f64(w1)
    bias = as_f64(b1)
    B, H = h.shape
    K = W1.shape[0]
    r = np.empty((B, K, H))
    for j in range(K):
        u = h @ W1[j].T + bias[j]          # u[b, i] = sum_c W1[j, i, c] * h[b, c] + b1[j, i]
        with np.errstate(over="ignore"):
            silu = u / (1.0 + np.exp(-u))
        r[:, j, :] = h + silu
    return r


def lm_head_logits(r, w_lm, head=None):
    """z[b, j, v] = sum_c Wlm[j, v, c] * r[b, j, c]  (no bias), float64.

    ``head`` selects one head (returns [B][V]); otherwise all heads [B][K][V].
    """
    if head is not None:
        W = as_f64(w_lm[head])
        return r[:, head, :] @ W.T
    K = w_lm.shape[0]
    return np.stack([r[:, j, :] @ as_f64(w_lm[j]).T for j in range(K)], axis=1)


def topk_by_value(z, k):
    """Indices of the k largest entries of each row of z.

    Order: value descending, then index ascending.  The comparison is taken
    on the float32-rounded values.  Returns (ids int32 [..., k], values
    float64 [..., k]) where the values are the unrounded float64 logits.
    """
    z = np.asarray(z, dtype=np.float64)
    lead = z.shape[:-1]
    V = z.shape[-1]
    flat = z.reshape(-1, V)
    ids = np.empty((flat.shape[0], k), dtype=np.int32)
    vals = np.empty((flat.shape[0], k))
    idx = np.arange(V)
    for row in range(flat.shape[0]):
        zf = flat[row].astype(np.float32)
        order = np.lexsort((idx, -zf.astype(np.float64)))  # primary key last: -value, then id
        ids[row] = order[:k]
        vals[row] = flat[row][order[:k]]
    return ids.reshape(lead + (k,)), vals.reshape(lead + (k,))


def heads(hidden, w1, b1, w_lm, topk, keep_logits=False):
    """All K heads: ResBlock, lm_head, top-k.

    Returns dict with r [B][K][H], topk_ids int32 [B][K][topk],
    topk_logits float64 [B][K][topk] and, with ``keep_logits``,
    logits [B][K][V].  The lm_head is evaluated one head at a time so the
    float64 copy of a head's weights is the largest temporary.
    """
    r = resblock(hidden, w1, b1)
    B, K, _ = r.shape
    ids = np.empty((B, K, topk), dtype=np.int32)
    vals = np.empty((B, K, topk))
    logits = [] if keep_logits else None
    for j in range(K):
        z = lm_head_logits(r, w_lm, head=j)   # [B][V]
        ids[:, j], vals[:, j] = topk_by_value(z, topk)
        if keep_logits:
            logits.append(z)
    out = dict(r=r, topk_ids=ids, topk_logits=vals)
    if keep_logits:
        out["logits"] = np.stack(logits, axis=1)
    return out
