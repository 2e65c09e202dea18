"""Pins for the oracle's tiny base model and its greedy decoding.

  * rmsnorm on a constant row has the closed form c / sqrt(c^2 + eps) * g;
  * RoPE with d = 2 is the plain 2-D rotation by the position (angle
    position * theta^0); it keeps every pair's norm, is the identity at
    position 0, and q(m).k(n) depends only on m - n;
  * with the blocks' output projections zero, every position's logits are
    lm_head . rmsnorm(embed[token]) (the residual stream is the embedding);
  * a one-layer model written with explicit loops over positions, heads and
    keys (its own causal softmax) gives the same logits;
  * causality: changing a later token leaves earlier logits unchanged;
  * greedy decoding of the zero-block model follows the token map
    f(x) = argmax lm_head . rmsnorm(embed[x]) computed by hand.
"""

import math

import numpy as np
import pytest

import oracle
import synth

D = oracle.decoder

CFG = dict(H=32, heads=2, I=48, layers=2, V=40, eps=1e-6, theta=10000.0)


def _model(cfg=CFG, seed=0):
    return synth.tiny_decoder(cfg, seed=seed)


def _f(x):
    return oracle.as_f64(x)


def test_rmsnorm_constant_row():
    g = np.array([1.0, 2.0, -0.5])
    for c in (3.0, -0.25):
        out = D.rmsnorm(np.full(3, c), g, 1e-6)
        assert np.allclose(out, c / math.sqrt(c * c + 1e-6) * g, rtol=1e-14)


def test_rope_two_dims_is_a_rotation():
    x = np.array([[[0.3, -1.2]]])          # [n=1][heads=1][d=2]
    for p in (0, 1, 5):
        out = D.rope(x, [p], 10000.0)[0, 0]
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(out, [0.3 * c + 1.2 * s, -1.2 * c + 0.3 * s], rtol=1e-14)


def test_rope_norm_identity_and_relative_positions():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    assert np.allclose(D.rope(q, [0], 10000.0), q, rtol=0, atol=1e-15)
    r = D.rope(q, [37], 10000.0)
    for i in range(8):
        assert math.isclose(r[0, 0, i] ** 2 + r[0, 0, i + 8] ** 2, q[0, 0, i] ** 2 + q[0, 0, i + 8] ** 2,
                            rel_tol=1e-12)
    dots = [float(np.sum(D.rope(q, [m], 10000.0) * D.rope(k, [m - 3], 10000.0))) for m in (3, 10, 50)]
    assert np.allclose(dots, dots[0], rtol=1e-10)


def _zero_blocks(model):
    m = dict(model, layers=[dict(l) for l in model["layers"]])
    for lw in m["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    return m


def test_zero_blocks_reduce_to_embedding_readout():
    m = _zero_blocks(_model())
    toks = [3, 17, 0, 39, 17]
    logits, _ = D.forward(m, toks)
    for i, t in enumerate(toks):
        h = _f(m["embed"])[t]
        hn = h / math.sqrt(np.mean(h * h) + CFG["eps"]) * _f(m["final_norm"])
        assert np.allclose(logits[i], _f(m["lm_head"]) @ hn, rtol=1e-12, atol=1e-12)


def _loop_forward(model, tokens):
    """One layer, explicit loops (own causal softmax and RoPE angles)."""
    cfg = model["cfg"]
    H, nh = cfg["H"], cfg["heads"]
    d, half = H // nh, H // nh // 2
    lw = model["layers"][0]
    n = len(tokens)

    def norm(v, g):
        return v / math.sqrt(sum(e * e for e in v) / len(v) + cfg["eps"]) * _f(g)

    def rot(vec, p):
        out = np.empty(d)
        for i in range(half):
            a = p * cfg["theta"] ** (-2.0 * i / d)
            out[i] = vec[i] * math.cos(a) - vec[i + half] * math.sin(a)
            out[i + half] = vec[i + half] * math.cos(a) + vec[i] * math.sin(a)
        return out

    xs = [_f(model["embed"])[t].copy() for t in tokens]
    a = [norm(x, lw["attn_norm"]) for x in xs]
    q = [[rot((_f(lw["wq"]) @ a[i])[h * d:(h + 1) * d], i) for h in range(nh)] for i in range(n)]
    k = [[rot((_f(lw["wk"]) @ a[i])[h * d:(h + 1) * d], i) for h in range(nh)] for i in range(n)]
    v = [[(_f(lw["wv"]) @ a[i])[h * d:(h + 1) * d] for h in range(nh)] for i in range(n)]
    out = []
    for i in range(n):
        o = np.zeros(H)
        for h in range(nh):
            sc = [float(q[i][h] @ k[j][h]) / math.sqrt(d) for j in range(i + 1)]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            o[h * d:(h + 1) * d] = sum(w[j] / tot * v[j][h] for j in range(i + 1))
        x = xs[i] + _f(lw["wo"]) @ o
        m = norm(x, lw["mlp_norm"])
        g = _f(lw["w_gate"]) @ m
        u = _f(lw["w_up"]) @ m
        x = x + _f(lw["w_down"]) @ (g / (1 + np.exp(-g)) * u)
        out.append(_f(model["lm_head"]) @ norm(x, model["final_norm"]))
    return np.array(out)


def test_one_layer_against_explicit_loops():
    cfg = dict(CFG, layers=1)
    m = _model(cfg, seed=3)
    toks = [5, 1, 33, 12, 5, 8]
    logits, _ = D.forward(m, toks)
    assert np.allclose(logits, _loop_forward(m, toks), rtol=1e-10, atol=1e-10)


def test_causality():
    m = _model(seed=4)
    a, _ = D.forward(m, [1, 2, 3, 4, 5])
    b, _ = D.forward(m, [1, 2, 3, 9, 0])
    assert np.allclose(a[:3], b[:3], rtol=0, atol=1e-12)
    assert not np.allclose(a[3], b[3])


def test_greedy_decoding_of_the_zero_block_model_follows_the_token_map():
    m = _zero_blocks(_model(seed=5))
    E, W, g = _f(m["embed"]), _f(m["lm_head"]), _f(m["final_norm"])
    f = [int(np.argmax(W @ (E[x] / math.sqrt(np.mean(E[x] ** 2) + CFG["eps"]) * g))) for x in range(CFG["V"])]
    toks, gaps = D.greedy_decode(m, [7], 12)
    expect, x = [], 7
    for _ in range(12):
        x = f[x]
        expect.append(x)
    assert toks == expect
    assert len(gaps) == 12 and min(gaps) > 0
