"""Seeded input tensors for each stage of the verify step.

All float tensors are drawn as float32 normals; bf16 workloads round them to
bf16 (nearest, ties to even) and return the uint16 bits.  Return values are
NumPy arrays in the layouts the library takes:

  hidden  [B][H]            w1 [K][H][H] (out x in)   b1 [K][H]
  w_lm    [K][V][H]         (out x in, no bias)
  q       [B][T][Hq][d]     k_cache, v_cache [B][Hq][S_max][d]
  logits  [B][T][V] fp32    cache  [n_layers][B][Hkv][S_max][d]
"""

import numpy as np

from .rng import stream, normal_f32, bf16_bits, f32_round


def _encode(x, dtype):
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return f32_round(x)
    raise ValueError(dtype)


def heads_inputs(w, seed=0, retries=None):
    """Hidden state and head weights for workload ``w``.

    Weights and b1 are N(0, 0.02^2); the hidden state is N(0, 1), divided by
    its root mean square when ``w['h_rms_norm']``.  ``retries[j]`` re-keys head
    j's lm_head stream (used to redraw a head whose top-k logits are too close
    together for a bit-exact comparison).
    """
    B, H, V, K = w["B"], w["H"], w["V"], w["K"]
    wid, dt = w["wid"], w["dtype"]
    retries = list(retries) if retries is not None else [0] * K
    h = normal_f32(seed, wid, "h", (), B * H).reshape(B, H)
    if w.get("h_rms_norm", False):
        h64 = h.astype(np.float64)
        h = (h64 / np.sqrt(np.mean(h64 * h64, axis=1, keepdims=True))).astype(np.float32)
    w1 = np.concatenate([normal_f32(seed, wid, "w1", (j,), H * H, std=0.02) for j in range(K)])
    b1 = normal_f32(seed, wid, "b1", (), K * H, std=0.02)
    wlm = np.concatenate([normal_f32(seed, wid, "wlm", (j, retries[j]), V * H, std=0.02)
                          for j in range(K)])
    return dict(
        hidden=_encode(h, dt).reshape(B, H),
        w1=_encode(w1, dt).reshape(K, H, H),
        b1=_encode(b1, dt).reshape(K, H),
        w_lm=_encode(wlm, dt).reshape(K, V, H),
        retries=retries,
    )


def topk_ids_input(w, seed=0):
    """int32 [B][K][topk]: distinct random token ids per (sequence, head)."""
    B, K, k, V = w["B"], w["K"], w["topk"], w["V"]
    out = np.empty((B, K, k), dtype=np.int32)
    for b in range(B):
        for j in range(K):
            g = stream(seed, w["wid"], "topk_ids", b, j)
            out[b, j] = g.choice(V, size=k, replace=False)
    return out


def root_token_input(w, seed=0):
    """int32 [B]: the base model's next token at the root of each tree."""
    g = stream(seed, w["wid"], "root")
    return g.integers(0, w["V"], size=w["B"], dtype=np.int64).astype(np.int32)


def prefix_lengths(w, seed=0):
    """int32 [B]: prefix length per sequence (fixed L, or uniform over L_range)."""
    if "L_range" in w:
        lo, hi = w["L_range"]
        g = stream(seed, w["wid"], "prefix")
        return g.integers(lo, hi + 1, size=w["B"], dtype=np.int64).astype(np.int32)
    return np.full(w["B"], w["L"], dtype=np.int32)


def rope_rotate(x, positions, theta=10000.0):
    """LLaMA rotate-half rotary embedding.

    ``x`` [..., n, d] float64 rows, ``positions`` [n] integer positions.
    Dims i and i + d/2 form a pair rotated by the angle p * theta^(-2i/d).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention_inputs(w, depth, prefix_len, seed=0, poison_tail=True, rope=True):
    """Queries and one layer of KV cache for tree attention.

    ``depth`` [T] is each tree node's depth in the caller's node order and
    ``prefix_len`` [B] the prefix per sequence.  Q, K, V are N(0, 1).  With
    ``rope``, prefix keys are rotated at their own slot positions and the tree
    queries and keys at prefix_len + depth.  Tree K/V sit at slots
    prefix_len .. prefix_len + T - 1.  With ``poison_tail`` every slot past the
    tree holds NaN, so any read of it shows up in the output.
    """
    B, Hq, d, S = w["B"], w["Hq"], w["d"], w["S_max"]
    T = len(depth)
    depth = np.asarray(depth, dtype=np.int64)
    wid, dt = w["wid"], w["dtype"]
    q = np.empty((B, T, Hq, d), dtype=np.float32)
    kc = np.zeros((B, Hq, S, d), dtype=np.float32)
    vc = np.zeros((B, Hq, S, d), dtype=np.float32)
    for b in range(B):
        L = int(prefix_len[b])
        if L + T > S:
            raise ValueError("prefix + tree exceeds the cache slots")
        qb = normal_f32(seed, wid, "q", (b,), T * Hq * d).reshape(T, Hq, d)
        kb = normal_f32(seed, wid, "k", (b,), Hq * (L + T) * d).reshape(Hq, L + T, d)
        vb = normal_f32(seed, wid, "v", (b,), Hq * (L + T) * d).reshape(Hq, L + T, d)
        if rope:
            pos_tree = L + depth
            pos_all = np.concatenate([np.arange(L), pos_tree])
            qb = rope_rotate(qb.transpose(1, 0, 2), pos_tree).transpose(1, 0, 2).astype(np.float32)
            kb = rope_rotate(kb, pos_all).astype(np.float32)
        q[b] = qb
        kc[b, :, :L + T] = kb
        vc[b, :, :L + T] = vb
        if poison_tail:
            kc[b, :, L + T:] = np.nan
            vc[b, :, L + T:] = np.nan
    return dict(q=_encode(q, dt), k_cache=_encode(kc, dt), v_cache=_encode(vc, dt))


def posterior_logits(w, tree_candidates=None, retrieve=None, num_paths=None, depth=None,
                     seed=0, gap=8.0, plant=None):
    """Base logits [B][T][V] fp32 at the tree nodes, N(0, logit_std^2).

    With ``plant`` (default ``w['planted']``) one deepest path per sequence
    is chosen uniformly, A ~ Binomial(depth, 1/2) is drawn, and for j < A the
    logit of the path's (j+1)-th token at its j-th node is set to that row's
    maximum plus ``gap``, so a greedy rule accepts exactly A tokens along it.
    The tree structure (``tree_candidates`` [B][T], ``retrieve`` [P][D],
    ``num_paths``, ``depth`` [T]) comes from the caller.  Returns
    (logits, plan) with plan[b] = (path index, A) or None.
    """
    B, V = w["B"], w["V"]
    plant = w.get("planted", False) if plant is None else plant
    T = len(depth) if depth is not None else int(np.asarray(tree_candidates).shape[1])
    out = np.empty((B, T, V), dtype=np.float32)
    plan = []
    for b in range(B):
        out[b] = normal_f32(seed, w["wid"], "logits", (b,), T * V,
                            std=w["logit_std"]).reshape(T, V)
        if not plant:
            plan.append(None)
            continue
        g = stream(seed, w["wid"], "plant", b)
        P = int(num_paths)
        ret = np.asarray(retrieve)[:P]
        lens = np.array([int(np.sum(r >= 0)) - 1 for r in ret])
        deepest = np.flatnonzero(lens == lens.max())
        p = int(deepest[int(g.integers(len(deepest)))])
        A = int(g.binomial(int(lens[p]), 0.5))
        for j in range(A):
            node = int(ret[p, j])
            tok = int(tree_candidates[b][int(ret[p, j + 1])])
            out[b, node, tok] = np.float32(float(out[b, node].max()) + gap)
        plan.append((p, A))
    return out, plan


def kv_cache(w, seed=0, n_layers=None, rows=None):
    """A bf16 (or f32) KV cache [n_layers][B][Hkv][S_max][d] of N(0, 1) values.

    ``rows`` limits the draw to slots [0, rows) (the rest stay zero).
    """
    nl = w["n_layers"] if n_layers is None else n_layers
    B, H, S, d = w["B"], w.get("Hkv", w["Hq"]), w["S_max"], w["d"]
    R = S if rows is None else int(rows)
    out = {}
    for name in ("cache_k", "cache_v"):
        x = np.zeros((nl, B, H, S, d), dtype=np.float32)
        x[:, :, :, :R] = normal_f32(seed, w["wid"], name, (), nl * B * H * R * d).reshape(nl, B, H, R, d)
        out[name] = _encode(x, w["dtype"])
    return out["cache_k"], out["cache_v"]


def base_head_inputs(M, H, V, seed=0, workload_id=9):
    """The base model's final hidden states at M tree nodes, N(0, 1), and its
    lm_head, N(0, 0.02^2), as bf16 bits: hidden [M][H], w_base [V][H]
    (out x in, no bias)."""
    h = normal_f32(seed, workload_id, "h_tree", (M, H), M * H)
    w = normal_f32(seed, workload_id, "w_base", (V, H), V * H, std=0.02)
    return dict(hidden=bf16_bits(h).reshape(M, H), w_base=bf16_bits(w).reshape(V, H))


def base_posterior_inputs(w, tree_candidates, retrieve, num_paths, seed=0, scale=7.0, plant=True, h_std=1.0):
    """Final hidden states at the tree nodes and a base lm_head, with one
    planted path per sequence (bf16 bits): hidden [B][T][H] ~ N(0, h_std^2),
    w_base [V][H] ~ N(0, 0.02^2), so a node's logits have standard deviation
    about 0.02 h_std sqrt(H) (h_std sets how peaked each node's distribution
    is, and with it the typical-acceptance thresholds).

    As in ``posterior_logits``, a deepest path is chosen uniformly and
    A ~ Binomial(depth, 1/2) drawn; for j < A, ``scale`` times the lm_head row
    of the path's (j+1)-th token is added to the hidden state of its j-th
    node, which lifts that token's logit there far above the row's others
    (by about scale * |w_row|^2).  Returns dict(hidden, w_base, plan).
    """
    B, H, V, wid = w["B"], w["H"], w["V"], w["wid"]
    cand = np.asarray(tree_candidates)
    T = int(cand.shape[1])
    wb = normal_f32(seed, wid, "w_base", (), V * H, std=0.02).reshape(V, H)
    h = normal_f32(seed, wid, "h_tree", (), B * T * H, std=h_std).reshape(B, T, H)
    plan = []
    for b in range(B):
        if not plant:
            plan.append(None)
            continue
        g = stream(seed, wid, "plant", b)
        P = int(num_paths)
        ret = np.asarray(retrieve)[:P]
        lens = np.array([int(np.sum(r >= 0)) - 1 for r in ret])
        deepest = np.flatnonzero(lens == lens.max())
        p = int(deepest[int(g.integers(len(deepest)))])
        A = int(g.binomial(int(lens[p]), 0.5))
        for j in range(A):
            node = int(ret[p, j])
            tok = int(cand[b][int(ret[p, j + 1])])
            h[b, node] += np.float32(scale) * wb[tok]
        plan.append((p, A))
    return dict(hidden=bf16_bits(h).reshape(B, T, H), w_base=bf16_bits(wb).reshape(V, H), plan=plan)


def node_uniforms(w, T, seed=0):
    """float32 [B][T] uniform variates in [0, 1): the random numbers a
    sampling acceptance mode draws with, one per tree node."""
    out = np.empty((w["B"], T), dtype=np.float32)
    for b in range(w["B"]):
        out[b] = stream(seed, w["wid"], "uniforms", b).random(T, dtype=np.float32)
    return out


def tiny_decoder(cfg, seed=0, workload_id=20):
    """Random weights of a tiny LLaMA-style base model (bf16 bits), out x in:
    embed [V][H] ~ N(0, 1); per layer wq, wk, wv [H][H] and w_gate, w_up
    [I][H] ~ N(0, 1/H), wo [H][H] ~ N(0, 0.25/H), w_down [H][I] ~ N(0,
    0.25/I); norm gains ~ 1 + N(0, 0.1^2); lm_head [V][H] ~ N(0, 4/H) (logits
    of standard deviation about 2).  cfg: H, heads, I, layers, V, eps, theta.
    """
    H, I, V = cfg["H"], cfg["I"], cfg["V"]

    def w(name, layer, shape, std, mean=0.0):
        n = int(np.prod(shape))
        return bf16_bits(normal_f32(seed, workload_id, "misc", (name, layer), n, std=std, mean=mean)).reshape(shape)

    names = {"embed": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "w_gate": 6, "w_up": 7, "w_down": 8,
             "attn_norm": 9, "mlp_norm": 10, "final_norm": 11, "lm_head": 12}
    layers = []
    for l in range(cfg["layers"]):
        layers.append(dict(
            attn_norm=w(names["attn_norm"], l, (H,), 0.1, 1.0),
            wq=w(names["wq"], l, (H, H), H ** -0.5), wk=w(names["wk"], l, (H, H), H ** -0.5),
            wv=w(names["wv"], l, (H, H), H ** -0.5), wo=w(names["wo"], l, (H, H), 0.5 * H ** -0.5),
            mlp_norm=w(names["mlp_norm"], l, (H,), 0.1, 1.0),
            w_gate=w(names["w_gate"], l, (I, H), H ** -0.5), w_up=w(names["w_up"], l, (I, H), H ** -0.5),
            w_down=w(names["w_down"], l, (H, I), 0.5 * I ** -0.5)))
    return dict(cfg=dict(cfg), embed=w(names["embed"], 0, (V, H), 1.0), layers=layers,
                final_norm=w(names["final_norm"], 0, (H,), 0.1, 1.0),
                lm_head=w(names["lm_head"], 0, (V, H), 2.0 * H ** -0.5))


def tiny_heads(cfg, K, seed=0, workload_id=21):
    """Random Medusa heads for the tiny model (bf16 bits): w1 [K][H][H],
    b1 [K][H] ~ N(0, 0.02^2); w_lm [K][V][H] ~ N(0, 4/H)."""
    H, V = cfg["H"], cfg["V"]
    return dict(w1=bf16_bits(normal_f32(seed, workload_id, "w1", (), K * H * H, std=0.02)).reshape(K, H, H),
                b1=bf16_bits(normal_f32(seed, workload_id, "b1", (), K * H, std=0.02)).reshape(K, H),
                w_lm=bf16_bits(normal_f32(seed, workload_id, "wlm", (), K * V * H, std=2.0 * H ** -0.5)).reshape(K, V, H))
