"""A tiny LLaMA-style base model and plain greedy decoding -- TEST
INFRASTRUCTURE ONLY.

The pages put Medusa heads on a decoder-only LLaMA-family model (Vicuna)
and verify the candidate tree with one forward of that model ([API]
tree_decoding; [NOTES] 核心要点); greedy Medusa decoding must emit exactly
what the base model's own greedy decoding emits ([NOTES] 学到什么: each
verify step keeps only what the base model would have produced).  The pages
do not spell the base model out; the reading taken is the LLaMA layer:

  x = embed[token]
  per layer:  x += Wo . attn(rope(Wq n), rope(Wk n), Wv n),  n = rmsnorm(x, g_attn)
              x += Wdown . (silu(Wgate n) * (Wup n)),        n = rmsnorm(x, g_mlp)
  hidden = rmsnorm(x, g_final);  logits = lm_head . hidden

rmsnorm(x, g) = x / sqrt(mean(x^2) + eps) * g; RoPE rotates dims i and
i + d/2 of each head by position * theta^(-2i/d); attention is causal
softmax(q.k / sqrt(d)) v per head.  Weights are stored out x in.

This module is the definition: every position is recomputed from the whole
sequence (no KV cache), in fp64 from the exact bf16 weight values.
"""

import numpy as np

from .attention import tree_attention
from .common import as_f64


def rmsnorm(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * as_f64(g)


def rope(x, positions, theta):
    """Rotate-half RoPE on the last axis of x [n][..][d] at positions [n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = float(theta) ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def forward(model, tokens):
    """Logits [n][V] and final hidden states [n][H] (fp64) of the sequence
    `tokens` at positions 0..n-1.  `model` holds cfg (H, heads, I, layers,
    V, eps, theta) and the bf16 weight arrays (see the module docstring)."""
    cfg = model["cfg"]
    H, nh = cfg["H"], cfg["heads"]
    d = H // nh
    tokens = [int(t) for t in tokens]
    n = len(tokens)
    pos = np.arange(n)
    x = as_f64(model["embed"])[tokens]                        # [n][H]
    causal = np.tril(np.ones((n, n), dtype=np.uint8))
    for lw in model["layers"]:
        a = rmsnorm(x, lw["attn_norm"], cfg["eps"])
        q = (a @ as_f64(lw["wq"]).T).reshape(n, nh, d)
        k = (a @ as_f64(lw["wk"]).T).reshape(n, nh, d)
        v = (a @ as_f64(lw["wv"]).T).reshape(n, nh, d)
        q, k = rope(q, pos, cfg["theta"]), rope(k, pos, cfg["theta"])
        # causal attention = tree attention with no prefix and a chain mask
        kc = np.ascontiguousarray(k.transpose(1, 0, 2))[None]  # [1][nh][n][d]
        vc = np.ascontiguousarray(v.transpose(1, 0, 2))[None]
        o = tree_attention(q[None], kc, vc, [0], causal, 1.0 / np.sqrt(d))[0]
        x = x + o.reshape(n, H) @ as_f64(lw["wo"]).T
        m = rmsnorm(x, lw["mlp_norm"], cfg["eps"])
        x = x + (silu(m @ as_f64(lw["w_gate"]).T) * (m @ as_f64(lw["w_up"]).T)) @ as_f64(lw["w_down"]).T
    hidden = rmsnorm(x, model["final_norm"], cfg["eps"])
    return hidden @ as_f64(model["lm_head"]).T, hidden


def greedy_decode(model, prompt, n_new):
    """The base model's own greedy continuation: n_new tokens, each the
    argmax (lowest id on ties) of the last position's logits over the whole
    sequence so far.  Returns (tokens, gaps): gaps[i] = the logit gap between
    the chosen token and the runner-up at step i."""
    seq = [int(t) for t in prompt]
    out, gaps = [], []
    for _ in range(n_new):
        logits, _ = forward(model, seq)
        z = logits[-1]
        t = int(np.argmax(z))
        gaps.append(float(z[t] - np.max(np.delete(z, t))))
        out.append(t)
        seq.append(t)
    return out, gaps
