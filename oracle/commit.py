"""Compaction of the accepted path's KV rows (test infrastructure only).

Definition followed: API reference page, ``tree_decoding`` (the tree tokens'
K/V are appended to ``past_key_values`` after the prefix) and study notes,
实践案例 案例 1 (only the accepted prefix of the best path is kept).  The
pages do not spell out the cache update; the reading taken is a gather with
snapshot semantics: slot L + j receives the row that was at slot
L + retrieve[best][j] before the update, for j = 0 .. accept_len (the root
included), and the new prefix length is L + accept_len + 1.  Slots past the
new prefix keep whatever they held.
"""

import numpy as np


def commit_kv(k_cache, v_cache, prefix_len, retrieve, best_path, accept_len):
    """New caches and prefix lengths.

    k_cache, v_cache [n_layers][B][H][S][d] (any element type, copied bit for
    bit); prefix_len, best_path, accept_len [B]; retrieve [P][D].
    Returns (new_k, new_v, new_prefix_len int64 [B]).
    """
    old_k = np.asarray(k_cache)
    old_v = np.asarray(v_cache)
    new_k = old_k.copy()
    new_v = old_v.copy()
    ret = np.asarray(retrieve)
    B = old_k.shape[1]
    new_len = np.zeros(B, dtype=np.int64)
    for b in range(B):
        L = int(prefix_len[b])
        path = ret[int(best_path[b])]
        a = int(accept_len[b])
        for j in range(a + 1):
            src = L + int(path[j])
            new_k[:, b, :, L + j] = old_k[:, b, :, src]
            new_v[:, b, :, L + j] = old_v[:, b, :, src]
        new_len[b] = L + a + 1
    return new_k, new_v, new_len
