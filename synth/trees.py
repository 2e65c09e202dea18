"""Tree specifications (``medusa_choices``): lists of rank tuples.

A rank tuple ``(r1, ..., rd)`` names the candidate reached by taking the
r1-th token of head 1, then the r2-th token of head 2, and so on.  These
helpers only *draw* specifications; ordering the nodes, finding parents and
building masks is the tree builder's job.
"""

import itertools

import numpy as np

from .rng import stream


def worked_example_choices():
    """Head 1 offers {A, B} (ranks 0, 1); head 2 offers {X, Y} after each of them."""
    return [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]


def full_tree_choices(K, topk):
    """Every rank tuple of length 1..K over range(topk) (a full topk-ary tree)."""
    out = []
    for depth in range(1, K + 1):
        out.extend(itertools.product(range(topk), repeat=depth))
    return [tuple(int(r) for r in t) for t in out]


def chain_choices(depth):
    """The chain (0,), (0, 0), ... of the given depth."""
    return [tuple([0] * d) for d in range(1, depth + 1)]


def random_tree_choices(depth_counts, max_children, seed=0, workload_id=0, shuffle=True):
    """A random tree with ``depth_counts[d-1]`` nodes at depth d.

    Depth-1 nodes hang off the root and take ranks 0, 1, ...  Every deeper
    node draws its parent uniformly among the previous depth's nodes; a parent
    that already has ``max_children`` children is drawn again.  A node's rank
    is its ordinal among its siblings in draw order.  Returns the tuples in
    draw order (shuffled when ``shuffle``), not in any canonical order.
    """
    g = stream(seed, workload_id, "tree", 0)
    if depth_counts[0] > max_children:
        raise ValueError("more depth-1 nodes than candidates per head")
    levels = [[(r,) for r in range(depth_counts[0])]]
    for count in depth_counts[1:]:
        prev = levels[-1]
        if count > len(prev) * max_children:
            raise ValueError("depth count exceeds the children available")
        nchild = [0] * len(prev)
        cur = []
        for _ in range(count):
            while True:
                p = int(g.integers(len(prev)))
                if nchild[p] < max_children:
                    break
            cur.append(prev[p] + (nchild[p],))
            nchild[p] += 1
        levels.append(cur)
    out = [t for lvl in levels for t in lvl]
    if shuffle:
        perm = g.permutation(len(out))
        out = [out[i] for i in perm]
    return out


def choices_array(choices, K):
    """int32 [N][K] array of rank tuples, padded with -1."""
    arr = np.full((len(choices), K), -1, dtype=np.int32)
    for i, t in enumerate(choices):
        if len(t) > K:
            raise ValueError("tuple longer than K")
        arr[i, :len(t)] = t
    return arr


# ------------------------------------------------------- tree-shape sweeps
# A synthetic acceptance model for choosing and scoring trees of a given
# size.  It is a workload model, not part of the verify step: it says how
# likely each head rank is to be the base model's next token.

def geometric_acceptance(K, topk, q1=0.85, gamma=0.9, rho=0.5):
    """p [K][topk]: p[d][i] = chance that rank i of head d+1 is the base
    model's token at that depth, given every earlier depth was right.
    Head d+1 holds q1 * gamma^d of that chance over its ranks, split
    geometrically with ratio rho: p[d][i] = q1 gamma^d (1 - rho) rho^i."""
    d = np.arange(K, dtype=np.float64)[:, None]
    i = np.arange(topk, dtype=np.float64)[None, :]
    return q1 * gamma ** d * (1.0 - rho) * rho ** i


def path_probability(p, t):
    """Chance that the whole rank tuple t is right: the product of its edges."""
    out = 1.0
    for depth, r in enumerate(t):
        out *= float(p[depth][r])
    return out


def best_tree_choices(p, n):
    """The n rank tuples of highest path probability (ties: the smaller
    tuple first), in that order.  Probabilities fall along both child and
    next-sibling edges (every p <= 1 and p[d] non-increasing in rank), so a
    best-first walk over those edges meets tuples in non-increasing order
    and the chosen set contains every chosen tuple's ancestors."""
    import heapq
    K, topk = len(p), len(p[0])
    heap = [(-path_probability(p, (0,)), (0,))]
    out = []
    while heap and len(out) < n:
        _, t = heapq.heappop(heap)
        out.append(t)
        if len(t) < K:
            c = t + (0,)
            heapq.heappush(heap, (-path_probability(p, c), c))
        if t[-1] + 1 < topk:
            s = t[:-1] + (t[-1] + 1,)
            heapq.heappush(heap, (-path_probability(p, s), s))
    if len(out) < n:
        raise ValueError("only %d tuples exist for K=%d, topk=%d" % (len(out), K, topk))
    return out


def expected_accept_length(p, choices):
    """Expected accepted length of a step on this tree: a step accepts
    exactly the tree nodes on the base model's own continuation (one token
    is right at each depth), so the mean is the sum of the nodes' path
    probabilities."""
    return float(sum(path_probability(p, t) for t in choices))
