"""Workload shapes for the Medusa verify step.

Each workload is a plain dict of sizes and rule parameters.  The Vicuna
shapes follow the LLaMA family the pages name (7B: hidden 4096, 32 heads of
128; 13B: hidden 5120, 40 heads of 128, 40 layers; 33B: hidden 6656, 52 heads
of 128, 60 layers; vocab 32000); K = 5 heads
is the pages' default head count.

Keys:
  dtype      "f32" or "bf16" for weights, hidden state and KV cache
  B          batch (independent sequences)
  H, V       hidden size, vocabulary size
  K, topk    Medusa heads, candidates kept per head
  tree       "full" (every rank tuple up to depth K) or "random" (depth counts)
  depth_counts  nodes per depth for the random tree (root excluded)
  Hq, d      attention heads and head dim for the tree-attention layer
  L          prefix length (scalar) or L_range (inclusive, drawn per sequence)
  n_layers   KV-cache layers touched by the commit
  S_max      cache slots per (layer, sequence, head)
  logit_std  std of the synthetic base logits at tree nodes
  planted    plant a greedy-accepted path (E[accepted] = depth/2)
  temperature, eps, delta   typical-acceptance parameters
"""

WORKLOADS = {
    # Tiny fp32 step: every stage at a size the oracle finishes instantly.
    "tiny-f32": dict(
        wid=0, dtype="f32", B=1, H=256, V=1000, K=3, topk=2, tree="full",
        Hq=4, d=64, L=128, n_layers=1, S_max=128 + 15,
        logit_std=3.0, planted=False, temperature=0.7, eps=0.09, delta=0.3,
        h_rms_norm=False,
    ),
    # Vicuna-7B verify step (batch 1).  The heads, the 64-node tree, one
    # attention layer at prefix 2048, the posterior over a 32000 vocab and the
    # 32-layer commit.
    "vicuna-7b": dict(
        wid=1, dtype="bf16", B=1, H=4096, V=32000, K=5, topk=10, tree="random",
        depth_counts=(10, 20, 16, 10, 7), Hq=32, d=128, L=2048,
        L_sweep=(512, 1024, 2048, 4096), n_layers=32, S_max=2048 + 64,
        logit_std=4.0, planted=True, temperature=0.7, eps=0.09, delta=0.3,
        h_rms_norm=True,
    ),
    # Vicuna-13B verify step (batch 1): hidden 5120, 40 heads of 128, 40 layers.
    "vicuna-13b": dict(
        wid=2, dtype="bf16", B=1, H=5120, V=32000, K=5, topk=10, tree="random",
        depth_counts=(10, 20, 16, 10, 7), Hq=40, d=128, L=2048, n_layers=40, S_max=2048 + 64,
        logit_std=4.0, planted=True, temperature=0.7, eps=0.09, delta=0.3,
        h_rms_norm=True,
    ),
    # Vicuna-33B, 8 independent sequences with their own prefixes.
    "vicuna-33b-b8": dict(
        wid=4, dtype="bf16", B=8, H=6656, V=32000, K=5, topk=10, tree="random",
        depth_counts=(10, 20, 16, 10, 7), Hq=52, d=128, L_range=(1024, 4096),
        n_layers=60, S_max=4096 + 64,
        logit_std=4.0, planted=True, temperature=0.7, eps=0.09, delta=0.3,
        h_rms_norm=True,
    ),
}


def workload(name, **overrides):
    """A copy of a named workload with some keys overridden."""
    w = dict(WORKLOADS[name])
    w["name"] = name
    w.update(overrides)
    return w
