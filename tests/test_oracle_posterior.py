"""Pins for the oracle's acceptance rule.

Greedy: a tiny random one-layer transformer is decoded token by token with
plain causal attention; verifying a random candidate tree with one tree-
masked forward and the greedy rule must accept exactly the longest prefix of
that greedy continuation present in the tree, and return the next greedy
token.  Typical: hand-built distributions whose entropy and threshold have
closed forms, temperature invariance, and the low-temperature limit.
"""

import math

import numpy as np
import pytest

import oracle
import synth


class TinyLM:
    """One attention head with RoPE and a residual, random weights."""

    def __init__(self, V, dm, seed):
        g = np.random.default_rng(seed)
        self.V, self.dm = V, dm
        self.E = g.standard_normal((V, dm))
        self.Wq = g.standard_normal((dm, dm)) / math.sqrt(dm)
        self.Wk = g.standard_normal((dm, dm)) / math.sqrt(dm)
        self.Wv = g.standard_normal((dm, dm)) / math.sqrt(dm)
        self.U = g.standard_normal((V, dm)) * 2.0
        self.scale = 1.0 / math.sqrt(dm)

    def qkv(self, tok, pos):
        x = self.E[tok]
        q = synth.rope_rotate((self.Wq @ x)[None], [pos])[0]
        k = synth.rope_rotate((self.Wk @ x)[None], [pos])[0]
        return x, q, k, self.Wv @ x

    def sequential_logits(self, tokens):
        """Logits after each token with plain causal attention (explicit loops)."""
        ks, vs, out = [], [], []
        for pos, tok in enumerate(tokens):
            x, q, k, v = self.qkv(tok, pos)
            ks.append(k)
            vs.append(v)
            s = [self.scale * float(q @ kk) for kk in ks]
            mx = max(s)
            e = [math.exp(a - mx) for a in s]
            att = sum(ei * vv for ei, vv in zip(e, vs)) / math.fsum(e)
            out.append(self.U @ (x + att))
        return out


def _greedy_continuation(lm, prefix, n):
    toks = list(prefix)
    logits = lm.sequential_logits(toks)
    ys = [int(np.argmax(logits[-1]))]          # the root: base model's next token
    for _ in range(n):
        logits = lm.sequential_logits(toks + ys)
        ys.append(int(np.argmax(logits[-1])))
    return ys


def _tree_forward(lm, prefix, t):
    """Base logits at every tree node from one tree-masked forward."""
    L = len(prefix)
    T = len(t["nodes"])
    cand = t["tree_candidates"][0]
    kc = np.zeros((1, 1, L + T, lm.dm))
    vc = np.zeros((1, 1, L + T, lm.dm))
    for pos, tok in enumerate(prefix):
        _, _, k, v = lm.qkv(tok, pos)
        kc[0, 0, pos], vc[0, 0, pos] = k, v
    q = np.zeros((1, T, 1, lm.dm))
    xs = []
    for i in range(T):
        x, qq, k, v = lm.qkv(int(cand[i]), int(t["position_ids"][0, i]))
        xs.append(x)
        q[0, i, 0] = qq
        kc[0, 0, L + i], vc[0, 0, L + i] = k, v
    att = oracle.tree_attention(q, kc, vc, np.array([L]), t["tree_mask"], lm.scale)[0, :, 0]
    return np.stack([lm.U @ (xs[i] + att[i]) for i in range(T)])


@pytest.mark.parametrize("seed", range(40))
def test_greedy_equals_sequential_decoding(seed):
    g = np.random.default_rng(1000 + seed)
    V, dm = 8, 12
    K = int(g.integers(1, 4))
    k = int(g.integers(1, 4))
    lm = TinyLM(V, dm, seed)
    prefix = [int(x) for x in g.integers(0, V, size=int(g.integers(2, 6)))]
    ys = _greedy_continuation(lm, prefix, K + 1)
    root = ys[0]
    # head j's candidates: k distinct tokens, containing the greedy token half the time
    topk = np.empty((1, K, k), dtype=np.int32)
    for j in range(K):
        ids = list(g.permutation(V)[:k])
        if ys[j + 1] not in ids and g.random() < 0.5:
            ids[int(g.integers(k))] = ys[j + 1]
        topk[0, j] = ids
    if g.random() < 0.5:
        choices = synth.full_tree_choices(K, k)
    else:
        counts = [min(k, int(g.integers(1, k + 1)))]
        for _ in range(K - 1):
            counts.append(int(g.integers(1, counts[-1] * k + 1)))
        choices = synth.random_tree_choices(counts, k, seed=seed)
    t = oracle.build_tree(synth.choices_array(choices, K), K, k, topk, np.array([root]),
                          np.array([len(prefix)]))
    logits = _tree_forward(lm, prefix, t)[None].astype(np.float32)
    res = oracle.evaluate_posterior(logits, t["tree_candidates"], t["retrieve"], t["num_paths"],
                                    0.0, 0.09, 0.3)
    # brute force: longest tree path spelling a prefix of the greedy continuation
    cand = t["tree_candidates"][0]
    best_len = 0
    for row in t["retrieve"][:t["num_paths"]]:
        n = 0
        for j in range(1, len(row)):
            if row[j] < 0 or int(cand[row[j]]) != ys[j]:
                break
            n += 1
        best_len = max(best_len, n)
    acc = int(res["accept_len"][0])
    assert acc == best_len
    path = t["retrieve"][int(res["best_path"][0])]
    assert [int(cand[path[j]]) for j in range(1, acc + 1)] == ys[1:acc + 1]
    assert int(res["next_token"][0]) == ys[acc + 1]


def _star(V, n_children, child_tokens, root_row, child_rows=None, temperature=1.0):
    """Root with n children (one path each); logits rows given per node."""
    T = 1 + n_children
    cand = np.array([[0] + list(child_tokens)], dtype=np.int32)
    retrieve = np.array([[0, 1 + c] for c in range(n_children)], dtype=np.int32)
    logits = np.zeros((1, T, V), dtype=np.float32)
    logits[0, 0] = root_row
    if child_rows is not None:
        logits[0, 1:] = child_rows
    return oracle.evaluate_posterior(logits, cand, retrieve, n_children, temperature, 0.09, 0.3)


def test_typical_uniform_accepts_everything():
    # uniform over V: H = ln V, threshold = min(0.09, 0.3/V) = 0.3/8 = 0.0375 < 1/8
    V, K, k = 8, 3, 2
    t = oracle.build_tree(synth.choices_array(synth.full_tree_choices(K, k), K), K, k,
                          np.arange(K * k, dtype=np.int32).reshape(1, K, k), np.array([7]),
                          np.array([0]))
    T = len(t["nodes"])
    logits = np.zeros((1, T, V), dtype=np.float32)
    res = oracle.evaluate_posterior(logits, t["tree_candidates"], t["retrieve"], t["num_paths"],
                                    1.0, 0.09, 0.3)
    st = res["stats"][0]
    assert np.allclose(st["H"], math.log(V), atol=1e-14)
    assert np.allclose(st["thr"], np.float32(0.3) / V, rtol=1e-7)
    assert res["accept_len"][0] == K and res["best_path"][0] == 0
    assert res["next_token"][0] == 0                      # first maximum of a flat row


def test_typical_dominant_token_only():
    # a gap of 60 leaves H ~ 0 and threshold 0.09: only the dominant token passes
    V = 10
    row = np.zeros(V, dtype=np.float32)
    row[4] = 60.0
    res = _star(V, 3, [4, 5, 6], row)
    assert res["stats"][0]["H"][0] < 1e-20
    assert res["path_len"][0].tolist() == [1, 0, 0]
    assert res["best_path"][0] == 0 and res["accept_len"][0] == 1


def test_typical_two_equal_tokens():
    # two tokens at p = 1/2: H = ln 2, threshold = min(0.09, 0.15) = 0.09: both pass
    V = 6
    row = np.full(V, -200.0, dtype=np.float32)
    row[[1, 3]] = 0.0
    res = _star(V, 3, [3, 1, 2], row)
    assert abs(res["stats"][0]["H"][0] - math.log(2.0)) < 1e-12
    assert res["path_len"][0].tolist() == [1, 1, 0]
    assert res["best_path"][0] == 0                        # several answers; lowest index wins


def test_typical_entropy_branch_binds():
    # 16 equal tokens: H = ln 16, threshold = 0.3/16 = 0.01875; p = 1/16 = 0.0625
    # lies below eps = 0.09 yet is accepted; a 17th token at p ~ 0 is rejected
    V = 40
    row = np.full(V, -300.0, dtype=np.float32)
    row[:16] = 1.5
    res = _star(V, 2, [17, 9], row)
    st = res["stats"][0]
    assert abs(st["H"][0] - math.log(16.0)) < 1e-12
    assert abs(st["thr"][0] - float(np.float32(0.3)) / 16) < 1e-12
    assert res["path_len"][0].tolist() == [0, 1]
    assert res["best_path"][0] == 1


@pytest.mark.parametrize("p,accepted", [(0.05, False), (0.10, True), (0.95, True)])
def test_typical_two_point(p, accepted):
    # distribution (p, 1-p): H = -p ln p - (1-p) ln(1-p) <= ln 2, so
    # 0.3 * exp(-H) >= 0.15 and the threshold is eps = 0.09
    V = 5
    row = np.full(V, -500.0, dtype=np.float32)
    row[0] = math.log(p)
    row[1] = math.log(1.0 - p)
    res = _star(V, 1, [0], row)
    H = -p * math.log(p) - (1 - p) * math.log(1 - p)
    assert abs(res["stats"][0]["H"][0] - H) < 1e-6
    assert abs(res["stats"][0]["thr"][0] - float(np.float32(0.09))) < 1e-12
    assert res["accept_len"][0] == (1 if accepted else 0)


@pytest.mark.parametrize("seed", range(5))
def test_temperature_invariance(seed):
    g = np.random.default_rng(seed)
    V, K, k = 30, 3, 3
    t = oracle.build_tree(synth.choices_array(synth.full_tree_choices(K, k), K), K, k,
                          g.integers(0, V, size=(1, K, k)).astype(np.int32), np.array([0]),
                          np.array([0]))
    T = len(t["nodes"])
    x = (g.standard_normal((1, T, V)) * 1.5).astype(np.float32)
    # make a few candidates likely so that some acceptances happen
    for i in range(1, T):
        x[0, t["parent"][i], t["tree_candidates"][0, i]] += float(g.choice([0.0, 4.0]))
    temp = 0.5
    a = oracle.evaluate_posterior(x, t["tree_candidates"], t["retrieve"], t["num_paths"], temp, 0.09, 0.3)
    b = oracle.evaluate_posterior((x.astype(np.float64) / np.float32(temp)).astype(np.float32),
                                  t["tree_candidates"], t["retrieve"], t["num_paths"], 1.0, 0.09, 0.3)
    assert np.array_equal(a["path_len"], b["path_len"])
    assert a["best_path"][0] == b["best_path"][0]


@pytest.mark.parametrize("seed", range(5))
def test_low_temperature_limit_is_greedy(seed):
    g = np.random.default_rng(50 + seed)
    V, K, k = 20, 3, 2
    t = oracle.build_tree(synth.choices_array(synth.full_tree_choices(K, k), K), K, k,
                          g.integers(0, V, size=(1, K, k)).astype(np.int32), np.array([0]),
                          np.array([0]))
    T = len(t["nodes"])
    x = g.standard_normal((1, T, V)).astype(np.float32)
    for n in range(T):
        x[0, n, int(np.argmax(x[0, n]))] += 1.0             # argmax margin >= 1
    for i in range(1, T):
        if g.random() < 0.6:
            row = x[0, t["parent"][i]]
            row[t["tree_candidates"][0, i]] = row.max() + 1.0
    greedy = oracle.evaluate_posterior(x, t["tree_candidates"], t["retrieve"], t["num_paths"], 0.0, 0.09, 0.3)
    cold = oracle.evaluate_posterior(x, t["tree_candidates"], t["retrieve"], t["num_paths"], 1e-3, 0.09, 0.3)
    assert np.array_equal(greedy["path_len"], cold["path_len"])
    assert greedy["next_token"][0] == cold["next_token"][0]


def test_padding_rejects_and_lowest_path_wins():
    # paths of different lengths; -1 padding ends a path
    V = 4
    cand = np.array([[0, 1, 2, 3]], dtype=np.int32)
    retrieve = np.array([[0, 1, -1], [0, 2, 3]], dtype=np.int32)
    x = np.zeros((1, 4, V), dtype=np.float32)
    x[0, 0, 1] = 5.0      # root prefers token 1 (node 1) ...
    x[0, 1, 0] = 5.0
    x[0, 2, 3] = 5.0      # node 2 would accept node 3, but node 2 itself is rejected
    res = oracle.evaluate_posterior(x, cand, retrieve, 2, 0.0, 0.09, 0.3)
    assert res["path_len"][0].tolist() == [1, 0]
    assert res["best_path"][0] == 0 and res["accept_len"][0] == 1
    assert res["next_token"][0] == 0                       # argmax at node 1
    x[0, 0, 1], x[0, 0, 2] = 0.0, 5.0
    res = oracle.evaluate_posterior(x, cand, retrieve, 2, 0.0, 0.09, 0.3)
    assert res["path_len"][0].tolist() == [0, 2]
    assert res["next_token"][0] == 0                       # node 3's row is flat


def test_typical_threshold_is_strict():
    # uniform over 8 tokens with eps = 1/8 and delta = 1: p = 1/8 and the
    # threshold min(1/8, exp(-ln 8)) rounds to 1/8 as well; p > thr fails.
    V = 8
    row = np.zeros(V, dtype=np.float32)
    cand = np.array([[0, 3]], dtype=np.int32)
    retrieve = np.array([[0, 1]], dtype=np.int32)
    x = np.zeros((1, 2, V), dtype=np.float32)
    x[0, 0] = row
    res = oracle.evaluate_posterior(x, cand, retrieve, 1, 1.0, 0.125, 1.0)
    assert float(np.float32(res["stats"][0]["thr"][0])) == 0.125
    assert res["accept_len"][0] == 0
    res = oracle.evaluate_posterior(x, cand, retrieve, 1, 1.0, 0.12, 1.0)
    assert res["accept_len"][0] == 1
