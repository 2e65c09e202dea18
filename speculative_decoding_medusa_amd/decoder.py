"""A LLaMA-style base model forward, plain greedy decoding and Medusa greedy
decoding, built from libmedusa calls.

This module only sequences library calls and keeps loop bookkeeping
(prefix lengths, the tokens a step emits); every computation runs in the
library's kernels.  The base model's layer is the one the C header
documents beside medusa_embed / medusa_add_rmsnorm / medusa_rope_qkv /
medusa_silu_mul; its linear layers run on medusa_linear (the base lm_head's
GEMM, its reduction split when the output is narrow) with weights packed
once.

Medusa greedy decoding ([API] medusa_generate, tree_decoding,
evaluate_posterior; [NOTES] 核心要点, 学到什么): the heads read the base
model's final hidden state at the last accepted token; the candidate tree,
rooted at the base model's own next token, runs through the base model in
one forward (tree tokens at positions prefix + depth, attending to the
prefix and their ancestors); the longest greedily accepted path and the
root are kept (their K/V moved into place), and the base model's token
after the last accepted node becomes the next root.  The emitted tokens are
exactly the base model's greedy continuation.

Sampled decoding (the pages' ``sampling='typical'`` with a positive
temperature, and the ``top_p`` nucleus mode): the same loop with the
typical acceptance test (medusa_evaluate_posterior at that temperature) and
a root -- the first token after the prompt, then each step's bonus token --
drawn by medusa_sample_typical, or with nucleus acceptance on the library's
Philox uniforms (medusa_philox_uniforms, medusa_evaluate_posterior_nucleus),
whose draw at the last accepted node is the next root.  Step s of a
generation draws with the keys (seed, s); the prompt's root is step 0.
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
        # workspaces of this decoder's own (never the binding's shared cache,
        # which a larger later call could reallocate under a captured graph)
        self.tmax = min(256, self.S)   # largest T one forward takes (prompt or tree)
        self.att_ws = torch.zeros(L.medusa_tree_attention_workspace(L.MEDUSA_BF16, 1, self.tmax, self.heads, self.d,
                                                                    self.S), dtype=torch.uint8, device=dev)
        self.post_ws = torch.zeros(L.medusa_posterior_workspace(1, self.tmax, self.V), dtype=torch.uint8, device=dev)
        # the projections' split-reduction partials (largest at 64 rows)
        H, I = self.H, self.I
        lin = max(L.medusa_linear_workspace(64, hin, vout)
                  for hin, vout in ((H, 3 * H), (H, H), (H, 2 * I), (I, H), (H, self.V)))
        self.lin_ws = torch.zeros(lin, dtype=torch.uint8, device=dev)
        # constants of the one-node acceptance test (argmax of one row)
        self._node0 = torch.zeros((1, 1), dtype=torch.int32, device=dev)
        self._npaths1 = torch.ones(1, dtype=torch.int32, device=dev)
        self._mask1 = torch.ones((1, 1), dtype=torch.uint8, device=dev)
        self._zero1 = torch.zeros(1, dtype=torch.int32, device=dev)
        self.nuc_ws = torch.zeros(L.medusa_posterior_nucleus_workspace(1, self.tmax), dtype=torch.uint8, device=dev)

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
            qkv = L.medusa_linear(n, lw["wqkv"], 3 * H, ws=self.lin_ws)
            q = L.medusa_rope_qkv(qkv.view(B, T, 3, self.heads, d), positions, prefix_len, self.theta,
                                  self.k_cache[l], self.v_cache[l])
            a = L.medusa_tree_attention(q, self.k_cache[l], self.v_cache[l], prefix_len, tree_mask, d ** -0.5,
                                        ws=self.att_ws)
            o = L.medusa_linear(a.view(B, T, H), lw["wo"], H, ws=self.lin_ws)
            n = L.medusa_add_rmsnorm(x, lw["mlp_norm"], self.eps, y=o)
            h = L.medusa_silu_mul(L.medusa_linear(n, lw["wgu"], 2 * I, ws=self.lin_ws))
            y = L.medusa_linear(h, lw["wdown"], H, ws=self.lin_ws)
        hidden = L.medusa_add_rmsnorm(x, self.final_norm, self.eps, y=y)
        return hidden, L.medusa_linear(hidden, self.lm_head, self.V, ws=self.lin_ws)

    # ------------------------------------------------------------ helpers
    def _i32(self, values, shape=None):
        t = torch.tensor(values, dtype=torch.int32).to(self.dev)
        return t.view(shape) if shape is not None else t

    def _argmax_last(self, logits):
        """The base model's greedy token at the last row of logits [1][T][V]
        (the acceptance test on a one-node tree), as a device int32 [1]."""
        row = logits[:, -1:, :]
        post = L.medusa_evaluate_posterior(row, self._node0, self._node0, self._npaths1, 0.0, 0.09, 0.3,
                                           ws=self.post_ws)
        return post["next_token"]

    def _sample_last(self, logits, mode, temperature, eps, delta, top_p, seed, step):
        """The sampled token at the last row of logits [1][T][V] under `mode`
        ('typical' or 'nucleus'), keys (seed, step), as a device int32 [1]."""
        row = logits[:, -1:, :]
        if mode == "typical":
            return L.medusa_sample_typical(row, self._node0, self._zero1, self._zero1, temperature, eps, delta, seed,
                                           step)
        if mode == "nucleus":
            u = L.medusa_philox_uniforms(seed, step, L.PURPOSE_NUCLEUS, 1, 1, device=self.dev)
            post = L.medusa_evaluate_posterior_nucleus(row, self._node0, self._node0, self._npaths1, temperature, top_p,
                                                       u, ws=self.nuc_ws)
            return post["next_token"]
        raise ValueError("mode must be 'typical' or 'nucleus'")

    def prefill(self, prompt):
        P = len(prompt)
        if not 1 <= P <= self.tmax:
            raise ValueError("prompt length must be in [1, %d]" % self.tmax)
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
        for i in range(1, n_new):
            Lp = P + i - 1
            _, logits = self.forward(nxt.view(1, 1), self._i32([[Lp]]), self._i32([Lp]), self._mask1)
            nxt = self._argmax_last(logits)
            toks.append(nxt)
        return [int(t) for t in torch.cat(toks).cpu()]

    def greedy_graph(self, prompt, n_new):
        """Plain greedy decoding with each step replayed from a HIP graph: the
        step (one-token forward, argmax, bookkeeping) keeps every value on the
        device -- the next token, its position, the prefix length and the
        output slot -- so the host only replays.  Same tokens as greedy()."""
        P = len(prompt)
        if P + n_new > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        if n_new < 2:
            return self.greedy(prompt, n_new)
        _, logits = self.prefill(prompt)
        tok = self._argmax_last(logits).clone().view(1, 1)
        pos = self._i32([[P]])
        plen = self._i32([P])
        idx = torch.zeros(1, dtype=torch.int64, device=self.dev)
        out = torch.empty(n_new, dtype=torch.int32, device=self.dev)
        out[:1].copy_(tok.view(1))

        def step():
            _, lg = self.forward(tok, pos, plen, self._mask1)
            nxt = self._argmax_last(lg)
            tok.view(1).copy_(nxt)
            pos.add_(1)
            plen.add_(1)
            idx.add_(1)
            out.scatter_(0, idx, nxt)

        step()   # the first step eagerly (also sizes every allocation)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(n_new - 2):
            graph.replay()
        return [int(t) for t in out.cpu()]

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
        tree = None
        while len(out) < n_new:
            r = L.medusa_resblock(h_row, heads["w1"], heads["b1"])
            ids = L.medusa_lm_head_topk(r, heads["w_lm"], topk, ws=ws)["topk_ids"]
            plen = self._i32([Lp])
            if tree is None:    # the tree's buffers once; each step gathers its candidates
                tree = L.medusa_build_tree(choices, ids, root, plen)
            else:
                L.medusa_tree_candidates(tree["tree_indices"], tree["depth"], ids, root, plen, out=tree)
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

    def medusa_graph(self, heads, choices, topk, prompt, n_new, check_every=4):
        """Medusa greedy decoding with each step replayed from a HIP graph.
        The step keeps its bookkeeping on the device: the emitted tokens
        (root and accepted nodes) are scattered into an output buffer at a
        device-side count, the next heads' input row is gathered at the last
        accepted node, the prefix length and root advance.  The host replays
        and reads the count every `check_every` steps.  Returns (tokens,
        steps)."""
        P = len(prompt)
        K = heads["w1"].shape[0]
        N = choices.shape[0]
        T = N + 1
        D = K + 1
        dev = self.dev
        slack = (check_every + 1) * D
        if P + n_new + slack + T > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        hidden, logits = self.prefill(prompt)
        root = self._argmax_last(logits).clone()
        h_row = hidden[:, P - 1, :].clone()
        plen = self._i32([P])
        new_plen = torch.empty(1, dtype=torch.int32, device=dev)
        cap = n_new + slack
        out = torch.zeros(cap + 1, dtype=torch.int32, device=dev)     # last slot: discarded writes
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        steps = torch.zeros(1, dtype=torch.int64, device=dev)
        jj = torch.arange(D, dtype=torch.int64, device=dev)
        trash = torch.full((D,), cap, dtype=torch.int64, device=dev)
        ws = torch.zeros(L.medusa_heads_workspace(L.MEDUSA_BF16, 1, self.H, self.V, K, topk), dtype=torch.uint8,
                         device=dev)
        i32 = torch.int32
        tree = dict(tree_candidates=torch.empty((1, T), dtype=i32, device=dev),
                    tree_indices=torch.empty(T, dtype=i32, device=dev), parent=torch.empty(T, dtype=i32, device=dev),
                    depth=torch.empty(T, dtype=i32, device=dev), position_ids=torch.empty((1, T), dtype=i32, device=dev),
                    tree_mask=torch.empty((T, T), dtype=torch.uint8, device=dev),
                    retrieve=torch.empty((T, D), dtype=i32, device=dev), num_paths=torch.empty(1, dtype=i32, device=dev),
                    status=torch.empty(2, dtype=i32, device=dev))
        post = {n: torch.empty(1, dtype=i32, device=dev) for n in ("best_path", "accept_len", "next_token")}
        r = torch.empty((1, K, self.H), dtype=torch.float32, device=dev)
        topk_out = dict(topk_ids=torch.zeros((1, K, topk), dtype=i32, device=dev),
                        topk_logits=torch.empty((1, K, topk), dtype=torch.float32, device=dev))

        # the tree's buffers once (its candidates are gathered every step)
        L.medusa_build_tree(choices, topk_out["topk_ids"], root, plen, out=tree)

        def step():
            L.medusa_resblock(h_row, heads["w1"], heads["b1"], r=r)
            L.medusa_lm_head_topk(r, heads["w_lm"], topk, out=topk_out, ws=ws)
            L.medusa_tree_candidates(tree["tree_indices"], tree["depth"], topk_out["topk_ids"], root, plen, out=tree)
            hid, lg = self.forward(tree["tree_candidates"], tree["position_ids"], plen, tree["tree_mask"])
            L.medusa_evaluate_posterior(lg, tree["tree_candidates"], tree["retrieve"], tree["num_paths"], 0.0, 0.09,
                                        0.3, out=post, ws=self.post_ws)
            L.medusa_commit_kv(self.k_cache, self.v_cache, plen, tree["retrieve"], post["best_path"],
                               post["accept_len"], new_prefix_len=new_plen)
            acc = post["accept_len"].long()
            path = tree["retrieve"].index_select(0, post["best_path"].long()).view(-1).long()   # [D]
            toks = tree["tree_candidates"].view(-1).index_select(0, path.clamp(min=0))
            dst = torch.where(jj <= acc, (count + jj).clamp(max=cap), trash)
            out.scatter_(0, dst, toks)
            count.add_(acc + 1)
            steps.add_(1)
            last = path.gather(0, acc)
            h_row.copy_(hid[0].index_select(0, last))
            plen.copy_(new_plen)
            root.copy_(post["next_token"])

        step()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        while True:
            if int(count.item()) >= n_new:
                break
            for _ in range(check_every):
                graph.replay()
        if int(tree["status"][0].item()) != 0:
            raise RuntimeError("tree spec rejected: %s" % tree["status"].cpu().tolist())
        return [int(t) for t in out[:n_new].cpu()], int(steps.item())

    # ------------------------------------------------------ sampled modes
    def sample(self, prompt, n_new, mode="typical", temperature=0.7, eps=0.09, delta=0.3, top_p=0.8, seed=0):
        """Plain sampled decoding, one token per forward: token i (i = 0 after
        the prompt) drawn under `mode` with keys (seed, i)."""
        P = len(prompt)
        if P + n_new > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        _, logits = self.prefill(prompt)
        nxt = self._sample_last(logits, mode, temperature, eps, delta, top_p, seed, 0)
        toks = [nxt]
        for i in range(1, n_new):
            Lp = P + i - 1
            _, logits = self.forward(nxt.view(1, 1), self._i32([[Lp]]), self._i32([Lp]), self._mask1)
            nxt = self._sample_last(logits, mode, temperature, eps, delta, top_p, seed, i)
            toks.append(nxt)
        return [int(t) for t in torch.cat(toks).cpu()]

    def medusa_sampled(self, heads, choices, topk, prompt, n_new, mode="typical", temperature=0.7, eps=0.09,
                       delta=0.3, top_p=0.8, seed=0, record=None):
        """Medusa decoding in a sampled mode: typical acceptance with a drawn
        bonus token ('typical'), or nucleus acceptance on Philox uniforms
        ('nucleus').  The prompt's root is drawn with keys (seed, 0), step s
        of the loop (s = 1, 2, ...) with (seed, s).  `record`, if a list,
        receives per step the host copies a caller needs to replay the
        step's decisions: logits [1][T][V], tree candidates, retrieve, path
        count, best path, accepted length, next root and the step index
        (step 0: the prompt's last logits row and the first root).
        Returns (tokens, accepted length per step)."""
        if mode not in ("typical", "nucleus"):
            raise ValueError("mode must be 'typical' or 'nucleus'")
        P = len(prompt)
        K = heads["w1"].shape[0]
        T = choices.shape[0] + 1
        if P + n_new + T > self.S:
            raise ValueError("the cache holds %d slots" % self.S)
        hidden, logits = self.prefill(prompt)
        root = self._sample_last(logits, mode, temperature, eps, delta, top_p, seed, 0)
        if record is not None:
            record.append(dict(step=0, logits=logits[:, -1:, :].cpu().numpy(), next_token=int(root[0])))
        h_row = hidden[:, P - 1, :]
        Lp = P
        out, accepts = [], []
        ws = torch.zeros(L.medusa_heads_workspace(L.MEDUSA_BF16, 1, self.H, self.V, K, topk), dtype=torch.uint8,
                         device=self.dev)
        tree = None
        s = 0
        while len(out) < n_new:
            s += 1
            r = L.medusa_resblock(h_row, heads["w1"], heads["b1"])
            ids = L.medusa_lm_head_topk(r, heads["w_lm"], topk, ws=ws)["topk_ids"]
            plen = self._i32([Lp])
            if tree is None:
                tree = L.medusa_build_tree(choices, ids, root, plen)
            else:
                L.medusa_tree_candidates(tree["tree_indices"], tree["depth"], ids, root, plen, out=tree)
            hidden, logits = self.forward(tree["tree_candidates"], tree["position_ids"], plen, tree["tree_mask"])
            if mode == "typical":
                post = L.medusa_evaluate_posterior(logits, tree["tree_candidates"], tree["retrieve"],
                                                   tree["num_paths"], temperature, eps, delta, ws=self.post_ws)
                nxt = L.medusa_sample_typical(logits, tree["retrieve"], post["best_path"], post["accept_len"],
                                              temperature, eps, delta, seed, s)
            else:
                u = L.medusa_philox_uniforms(seed, s, L.PURPOSE_NUCLEUS, 1, T, device=self.dev)
                post = L.medusa_evaluate_posterior_nucleus(logits, tree["tree_candidates"], tree["retrieve"],
                                                           tree["num_paths"], temperature, top_p, u, ws=self.nuc_ws)
                nxt = post["next_token"]
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
            if record is not None:
                record.append(dict(step=s, logits=logits.cpu().numpy(), tree_candidates=np.array([cand], np.int32),
                                   retrieve=tree["retrieve"].cpu().numpy(), num_paths=int(tree["num_paths"][0]),
                                   best_path=best, accept_len=acc, next_token=int(nxt[0])))
            h_row = hidden[:, path[acc], :]
            Lp += acc + 1
            root = nxt.clone()
        return out[:n_new], accepts
