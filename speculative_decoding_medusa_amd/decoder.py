"""A LLaMA-style base model forward, plain greedy decoding and Medusa greedy
decoding, built from libmedusa calls.

This module only sequences library calls and keeps loop bookkeeping
(prefix lengths, the tokens a step emits); every computation runs in the
library's kernels.  The base model's layer is the one the C header
documents beside medusa_embed / medusa_add_rmsnorm / medusa_rope_qkv /
medusa_silu_mul; its linear layers run on medusa_base_lm_head with weights
packed once.

Medusa greedy decoding ([API] medusa_generate, tree_decoding,
evaluate_posterior; [NOTES] 核心要点, 学到什么): the heads read the base
model's final hidden state at the last accepted token; the candidate tree,
rooted at the base model's own next token, runs through the base model in
one forward (tree tokens at positions prefix + depth, attending to the
prefix and their ancestors); the longest greedily accepted path and the
root are kept (their K/V moved into place), and the base model's token
after the last accepted node becomes the next root.  The emitted tokens are
exactly the base model's greedy continuation.
"""

import numpy as np
import torch

from . import _lib as L


def _bf16(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("weights are bf16 bit patterns (uint16)")
    return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)


class TinyDecoder:
    """Weights (bf16 bits, out x in) and a KV cache of `max_slots` slots on
    one device; batch 1.  `model` = dict(cfg=dict(H, heads, I, layers, V,
    eps, theta), embed, layers=[dict(attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate, w_up, w_down)], final_norm, lm_head)."""

    def __init__(self, model, device, max_slots):
        cfg = model["cfg"]
        self.cfg = cfg
        self.H, self.heads, self.I, self.V = cfg["H"], cfg["heads"], cfg["I"], cfg["V"]
        self.d = self.H // self.heads
        self.eps, self.theta = float(cfg["eps"]), float(cfg["theta"])
        self.S = int(max_slots)
        dev = torch.device(device)
        self.dev = dev

        def pack(w):
            return L.medusa_base_lm_head_pack(_bf16(w, dev))

        self.embed = _bf16(model["embed"], dev)
        self.layers = []
        for lw in model["layers"]:
            self.layers.append(dict(
                attn_norm=_bf16(lw["attn_norm"], dev), mlp_norm=_bf16(lw["mlp_norm"], dev),
                wqkv=pack(np.concatenate([lw["wq"], lw["wk"], lw["wv"]])), wo=pack(lw["wo"]),
                wgu=pack(np.concatenate([lw["w_gate"], lw["w_up"]])), wdown=pack(lw["w_down"])))
        self.final_norm = _bf16(model["final_norm"], dev)
        self.lm_head = pack(model["lm_head"])
        shape = (len(self.layers), 1, self.heads, self.S, self.d)
        self.k_cache = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        self.v_cache = torch.zeros(shape, dtype=torch.bfloat16, device=dev)

    def forward(self, tokens, positions, prefix_len, tree_mask):
        """Run tokens [1][T] (int32, device) at positions [1][T] against the
        cache prefix [0, prefix_len) plus, for token i, the tokens j with
        tree_mask[i][j] = 1 (their K/V written to slots prefix_len + j of
        every layer).  Returns (hidden bf16 [1][T][H] after the final norm,
        logits float32 [1][T][V])."""
        B, T = tokens.shape
        H, I, d = self.H, self.I, self.d
        x = L.medusa_embed(tokens, self.embed)
        y = None
        for l, lw in enumerate(self.layers):
            n = L.medusa_add_rmsnorm(x, lw["attn_norm"], self.eps, y=y)
            qkv = L.medusa_base_lm_head(n, lw["wqkv"], V=3 * H)
            q = L.medusa_rope_qkv(qkv.view(B, T, 3, self.heads, d), positions, prefix_len, self.theta,
                                  self.k_cache[l], self.v_cache[l])
            a = L.medusa_tree_attention(q, self.k_cache[l], self.v_cache[l], prefix_len, tree_mask, d ** -0.5)
            o = L.medusa_base_lm_head(a.view(B, T, H), lw["wo"], V=H)
            n = L.medusa_add_rmsnorm(x, lw["mlp_norm"], self.eps, y=o)
            h = L.medusa_silu_mul(L.medusa_base_lm_head(n, lw["wgu"], V=2 * I))
            y = L.medusa_base_lm_head(h, lw["wdown"], V=H)
        hidden = L.medusa_add_rmsnorm(x, self.final_norm, self.eps, y=y)
        return hidden, L.medusa_base_lm_head(hidden, self.lm_head, V=self.V)

    # ------------------------------------------------------------ helpers
    def _i32(self, values, shape=None):
        t = torch.tensor(values, dtype=torch.int32).to(self.dev)
        return t.view(shape) if shape is not None else t

    def _argmax_last(self, logits):
        """The base model's greedy token at the last row of logits [1][T][V]
        (the acceptance test on a one-node tree), as a device int32 [1]."""
        row = logits[:, -1:, :]
        one = self._i32([[0]])
        post = L.medusa_evaluate_posterior(row, one.view(1, 1), one, self._i32([1]), 0.0, 0.09, 0.3)
        return post["next_token"]

    def prefill(self, prompt):
        P = len(prompt)
        if not 1 <= P <= 256:
            raise ValueError("prompt length must be in [1, 256]")
        mask = torch.tril(torch.ones((P, P), dtype=torch.uint8)).to(self.dev)
        hidden, logits = self.forward(self._i32([list(prompt)]), self._i32([list(range(P))]), self._i32([0]), mask)
        return hidden, logits

    # --------------------------------------------------------- generation
    def greedy(self, prompt, n_new):
        """Plain greedy decoding: one token per forward.  Returns the n_new
        tokens."""
        P = len(prompt)
        if P + n_new > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        _, logits = self.prefill(prompt)
        nxt = self._argmax_last(logits)
        toks = [nxt]
        one = torch.ones((1, 1), dtype=torch.uint8, device=self.dev)
        for i in range(1, n_new):
            Lp = P + i - 1
            _, logits = self.forward(nxt.view(1, 1), self._i32([[Lp]]), self._i32([Lp]), one)
            nxt = self._argmax_last(logits)
            toks.append(nxt)
        return [int(t) for t in torch.cat(toks).cpu()]

    def medusa(self, heads, choices, topk, prompt, n_new):
        """Medusa greedy decoding with heads = dict(w1 [K][H][H], b1 [K][H],
        w_lm [K][V][H]) (bf16 device tensors) and a medusa_choices spec
        (int32 [N][K] device).  Returns (tokens, accepted length per step,
        best path per step)."""
        P = len(prompt)
        K = heads["w1"].shape[0]
        T = choices.shape[0] + 1
        if P + n_new + T > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        hidden, logits = self.prefill(prompt)
        root = self._argmax_last(logits)
        h_row = hidden[:, P - 1, :]
        Lp = P
        out, accepts, paths = [], [], []
        ws = torch.zeros(L.medusa_heads_workspace(L.MEDUSA_BF16, 1, self.H, self.V, K, topk), dtype=torch.uint8,
                         device=self.dev)
        while len(out) < n_new:
            r = L.medusa_resblock(h_row, heads["w1"], heads["b1"])
            ids = L.medusa_lm_head_topk(r, heads["w_lm"], topk, ws=ws)["topk_ids"]
            plen = self._i32([Lp])
            tree = L.medusa_build_tree(choices, ids, root, plen)
            hidden, logits = self.forward(tree["tree_candidates"], tree["position_ids"], plen, tree["tree_mask"])
            post = L.medusa_evaluate_posterior(logits, tree["tree_candidates"], tree["retrieve"], tree["num_paths"],
                                               0.0, 0.09, 0.3)
            L.medusa_commit_kv(self.k_cache, self.v_cache, plen, tree["retrieve"], post["best_path"],
                               post["accept_len"])
            status = tree["status"].cpu().tolist()
            if status[0] != 0:
                raise RuntimeError("tree spec rejected: %s" % status)
            best, acc = int(post["best_path"][0]), int(post["accept_len"][0])
            path = tree["retrieve"][best].cpu().tolist()
            cand = tree["tree_candidates"][0].cpu().tolist()
            out.extend(cand[path[j]] for j in range(acc + 1))
            accepts.append(acc)
            paths.append(best)
            h_row = hidden[:, path[acc], :]
            Lp += acc + 1
            root = post["next_token"]
        return out[:n_new], accepts, paths
