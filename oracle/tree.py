"""Candidate tree from a ``medusa_choices`` spec (test infrastructure only).

Definition followed:
  * API reference page, ``medusa_generate`` (the ``medusa_choices``
    argument), ``generate_candidates`` (``tree_indices``,
    ``retrieve_indices``) and ``tree_decoding`` (``tree_candidates``,
    ``medusa_position_ids``).
  * Study notes, 核心要点 (tree attention: the per-head top-k tokens form a
    prefix tree) and 实践案例 案例 3 (the worked mask: with head-1 tokens
    {A, B} and head-2 tokens {X, Y}, the forward input is P, A, B, X, Y, X, Y;
    the X that follows A sees only P and A, the X that follows B only P and B).

A spec entry is a rank tuple (r1, ..., rd): the r1-th token of head 1, then
the r2-th token of head 2, and so on.  Readings where the pages are silent:
nodes are ordered root first, then by (depth, rank tuple in lexicographic
order), which reproduces the worked example's order; tree_indices index the
flat list [root token, head-1 top-k, head-2 top-k, ...]; position ids are
prefix length + depth; a node attends to its ancestors and itself; leaves in
ascending node order give the retrieve paths, padded with -1.
"""

import numpy as np


class SpecError(ValueError):
    """A malformed spec.  ``kind`` is one of: 'padding', 'empty', 'rank',
    'duplicate', 'prefix', 'too_many_paths'."""

    def __init__(self, kind, index):
        super().__init__("%s (entry %d)" % (kind, index))
        self.kind = kind
        self.index = index


def parse_choices(choices, topk):
    """Rank tuples from an int32 [N][K] array padded with -1.

    Checks, entry by entry in the given order: padding is a -1 suffix,
    the tuple is not empty, every rank lies in [0, topk); then no tuple
    repeats and every proper prefix of a tuple is itself an entry.
    """
    arr = np.asarray(choices)
    tuples = []
    for i, row in enumerate(arr):
        row = [int(x) for x in row]
        n = len(row)
        while n > 0 and row[n - 1] == -1:
            n -= 1
        t = row[:n]
        if any(x == -1 for x in t):
            raise SpecError("padding", i)
        if n == 0:
            raise SpecError("empty", i)
        if any(x < 0 or x >= topk for x in t):
            raise SpecError("rank", i)
        tuples.append(tuple(t))
    seen = {}
    for i, t in enumerate(tuples):
        if t in seen:
            raise SpecError("duplicate", i)
        seen[t] = i
    for i, t in enumerate(tuples):
        for m in range(1, len(t)):
            if t[:m] not in seen:
                raise SpecError("prefix", i)
    return tuples


def build_tree(choices, K, topk, topk_ids, root_token, prefix_len, p_max=None):
    """The tree for one spec, shared by every sequence of the batch.

    choices [N][K] int32 (-1 padded), topk_ids [B][K][topk], root_token [B],
    prefix_len [B].  Returns a dict of NumPy arrays:
      nodes            list of rank tuples, node 0 = () the root
      tree_candidates  int32 [B][T]   token at each node
      tree_indices     int32 [T]      index into [root, head1 top-k, head2 top-k, ...]
      parent, depth    int32 [T]      parent[0] = -1
      position_ids     int32 [B][T]   prefix_len + depth
      tree_mask        uint8 [T][T]   1 where column j is an ancestor of row i or i itself
      retrieve         int32 [P][K+1] root-to-leaf node lists, -1 padded
      num_paths        int            P
    """
    tuples = parse_choices(choices, topk)
    nodes = [()] + sorted(tuples, key=lambda t: (len(t), t))
    T = len(nodes)
    index = {t: i for i, t in enumerate(nodes)}
    depth = np.array([len(t) for t in nodes], dtype=np.int32)
    parent = np.array([-1] + [index[t[:-1]] for t in nodes[1:]], dtype=np.int32)
    tree_indices = np.array([0] + [1 + (len(t) - 1) * topk + t[-1] for t in nodes[1:]],
                            dtype=np.int32)

    topk_ids = np.asarray(topk_ids)
    B = topk_ids.shape[0]
    tree_candidates = np.empty((B, T), dtype=np.int32)
    position_ids = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        flat = [int(root_token[b])] + [int(x) for x in topk_ids[b].reshape(-1)]
        for i in range(T):
            tree_candidates[b, i] = flat[tree_indices[i]]
            position_ids[b, i] = int(prefix_len[b]) + depth[i]

    mask = np.zeros((T, T), dtype=np.uint8)
    for i, ti in enumerate(nodes):
        for j, tj in enumerate(nodes):
            if ti[:len(tj)] == tj:       # tj is a prefix of ti (the root () of everything)
                mask[i, j] = 1

    has_child = np.zeros(T, dtype=bool)
    has_child[parent[1:]] = True
    leaves = [i for i in range(T) if not has_child[i]]
    if p_max is not None and len(leaves) > p_max:
        raise SpecError("too_many_paths", len(leaves))
    D = K + 1
    retrieve = np.full((len(leaves), D), -1, dtype=np.int32)
    for p, leaf in enumerate(leaves):
        t = nodes[leaf]
        for m in range(len(t) + 1):
            retrieve[p, m] = index[t[:m]]

    return dict(nodes=nodes, tree_candidates=tree_candidates, tree_indices=tree_indices,
                parent=parent, depth=depth, position_ids=position_ids, tree_mask=mask,
                retrieve=retrieve, num_paths=len(leaves))
