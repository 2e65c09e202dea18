"""Tree-masked attention over a KV prefix (test infrastructure only).

Definition followed:
  * Study notes, 核心要点 (tree attention: one forward verifies every
    candidate continuation, a mask keeping each continuation to its own
    branch) and 实践案例 案例 3 (each tree token sees the prompt and its own
    ancestors only).
  * API reference page, ``tree_decoding``: the tree tokens are run against
    ``past_key_values`` (the KV cache of the prefix).

Reading where the pages are silent: plain softmax attention with scale
1/sqrt(d) applied by the caller's ``scale``; queries and tree keys arrive
already position-encoded (the positions being prefix length + depth); the
tree's K/V rows sit in the cache right after the prefix.
"""

import numpy as np

from .common import as_f64


def tree_attention(q, k_cache, v_cache, prefix_len, tree_mask, scale):
    """out[b, i, h] = softmax_m(scale * q[b,i,h] . k[b,h,m]) @ v[b,h,m].

    The keys m of query i are the prefix slots 0..L-1 and the tree slots
    L + j for every node j with tree_mask[i][j] = 1 (L = prefix_len[b]).

    q [B][T][Hq][d]; k_cache, v_cache [B][Hq][S][d]; tree_mask [T][T].
    Returns float64 [B][T][Hq][d].
    """
    Q = as_f64(q)
    B, T, Hq, d = Q.shape
    mask = np.asarray(tree_mask).astype(bool)
    out = np.empty((B, T, Hq, d))
    for b in range(B):
        L = int(prefix_len[b])
        Kb = as_f64(k_cache[b, :, :L + T])   # [Hq][L+T][d]
        Vb = as_f64(v_cache[b, :, :L + T])
        allowed = np.concatenate([np.ones((T, L), dtype=bool), mask], axis=1)  # [T][L+T]
        for h in range(Hq):
            s = (Q[b, :, h, :] @ Kb[h].T) * float(scale)          # [T][L+T]
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ Vb[h]
    return out
