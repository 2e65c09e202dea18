"""Pins for the oracle's KV commit.

Brute force: the compacted cache's first new_L slots must equal the prefix
followed by the accepted path's rows appended one by one; a chain path is the
identity; overlapping source/destination slots follow snapshot semantics.
"""

import numpy as np
import pytest

import oracle


def _cache(nl, B, H, S, d, seed):
    g = np.random.default_rng(seed)
    return (g.integers(0, 1 << 16, size=(nl, B, H, S, d)).astype(np.uint16),
            g.integers(0, 1 << 16, size=(nl, B, H, S, d)).astype(np.uint16))


@pytest.mark.parametrize("seed", range(6))
def test_commit_equals_sequential_append(seed):
    g = np.random.default_rng(seed)
    nl, B, H, d = 3, 2, 2, 4
    T, D = 9, 4
    L = g.integers(2, 6, size=B)
    S = int(L.max()) + T + 2
    kc, vc = _cache(nl, B, H, S, d, seed)
    # three paths through a 9-node tree (node ids increase along a path)
    retrieve = np.array([[0, 1, 4, 7], [0, 2, 5, -1], [0, 3, 6, 8]], dtype=np.int32)
    best = g.integers(0, 3, size=B)
    acc = np.array([g.integers(0, int(np.sum(retrieve[p] >= 0))) for p in best])
    nk, nv, nlen = oracle.commit_kv(kc, vc, L, retrieve, best, acc)
    for b in range(B):
        Lb = int(L[b])
        rows = [Lb + int(retrieve[best[b], j]) for j in range(acc[b] + 1)]
        want_k = np.concatenate([kc[:, b, :, :Lb], kc[:, b][:, :, rows]], axis=2)
        want_v = np.concatenate([vc[:, b, :, :Lb], vc[:, b][:, :, rows]], axis=2)
        assert nlen[b] == Lb + acc[b] + 1
        assert np.array_equal(nk[:, b, :, :nlen[b]], want_k)
        assert np.array_equal(nv[:, b, :, :nlen[b]], want_v)
        # slots past the new prefix are left as they were
        assert np.array_equal(nk[:, b, :, nlen[b]:], kc[:, b, :, nlen[b]:])


def test_chain_path_is_identity():
    kc, vc = _cache(2, 1, 3, 20, 4, 1)
    retrieve = np.array([[0, 1, 2, 3]], dtype=np.int32)
    nk, nv, nlen = oracle.commit_kv(kc, vc, np.array([10]), retrieve, np.array([0]), np.array([3]))
    assert np.array_equal(nk, kc) and np.array_equal(nv, vc)
    assert nlen.tolist() == [14]


def test_overlap_snapshot_semantics():
    # path (0, 2, 11) with two accepted: slot L+1 <- old L+2, slot L+2 <- old L+11
    kc, vc = _cache(1, 1, 1, 30, 2, 2)
    L = 5
    retrieve = np.array([[0, 2, 11, -1]], dtype=np.int32)
    nk, _, nlen = oracle.commit_kv(kc, vc, np.array([L]), retrieve, np.array([0]), np.array([2]))
    got = nk[0, 0, 0, L:L + 3]
    want = np.stack([kc[0, 0, 0, L], kc[0, 0, 0, L + 2], kc[0, 0, 0, L + 11]])
    assert np.array_equal(got, want)
    assert nlen.tolist() == [L + 3]
