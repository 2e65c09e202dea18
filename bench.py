"""Benchmark: Medusa verify steps per second at the Vicuna-7B shape (batch 1).

One step = every stage of the verify step on one HIP stream:
  ResBlock (5 heads, H 4096)  ->  lm_head + top-10 (5 x 32000 x 4096 bf16)
  -> candidate tree (64 nodes: built once per tree spec, this step's
  candidates and positions gathered through it)  ->  tree attention (32 heads x 128, prefix
  2048, one layer; the layer rotates over the 32-layer cache)
  -> typical acceptance (T 0.7, eps 0.09, delta 0.3) over [64][32000] logits
  -> KV commit across 32 layers x 32 heads.
Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --tree-sweep [--steps K]     # step cost vs heads K and tree size T
    python bench.py --generate                   # end-to-end greedy generation, plain vs Medusa

Prints one JSON line.  `roofline` covers the dominant kernel (lm_head +
top-k): algorithmic bytes per launch over its mean duration, measured with
HIP events on the stream it runs on.  `cpu_baseline` times the CPU oracle on
one full step on this host.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Medusa verify steps/sec at Vicuna-7B shape (batch 1); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
LM_SAMPLE = 10   # the roofline call is bracketed by events in one timed step of every LM_SAMPLE
SETTLE_MS = 30.0 # GPU time of untimed steps before the warm-up
STAGE_STEPS = 200  # steps of the untimed per-stage breakdown pass


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-base-head", action="store_true",
                    help="skip the base lm_head timing (the step before the acceptance test)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the tree-attention prefix sweep and the Vicuna-33B batch-8 legs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device-to-device copy of COPY_PROBE_BYTES (counter calibration)")
    ap.add_argument("--generate", action="store_true",
                    help="run only end-to-end generation on a small LLaMA-style model: plain greedy against "
                         "Medusa greedy (one JSON line)")
    ap.add_argument("--attention", type=int, default=0, metavar="L",
                    help="run only tree attention (64-node tree, 32 x 128 heads) at prefix L, --steps calls over "
                         "eight rotated layers (for kernel traces and counters; one JSON line)")
    ap.add_argument("--tree-sweep", action="store_true",
                    help="run only the tree-shape sweep: step cost and expected tokens per step against the "
                         "number of heads K and tree nodes T (one JSON line)")
    return ap.parse_args()


COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """A plain copy of a known size, three times: what FETCH_SIZE / WRITE_SIZE
    read for it calibrates the counters against the bytes really moved."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 3}))


class Step:
    """All buffers and pre-marshalled arguments of one verify step."""

    NLOGITS = 64

    def __init__(self, w, seed):
        import numpy as np
        import torch

        import speculative_decoding_medusa_amd as md
        import synth

        self.md, self.torch = md, torch
        dev = torch.device("cuda:0")
        self.dev = dev
        self.w = w
        self.stream = torch.cuda.current_stream(dev).cuda_stream

        def d(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        B, H, V, K, k = w["B"], w["H"], w["V"], w["K"], w["topk"]
        x = synth.heads_inputs(w, seed=seed)
        self.hidden, self.w1, self.b1, self.w_lm = (d(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
        del x
        self.r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
        self.topk_ids = torch.empty((B, K, k), dtype=torch.int32, device=dev)
        self.topk_vals = torch.empty((B, K, k), dtype=torch.float32, device=dev)
        self.heads_ws = torch.zeros(md.medusa_heads_workspace(md.MEDUSA_BF16, B, H, V, K, k),
                                    dtype=torch.uint8, device=dev)

        choices = synth.random_tree_choices(w["depth_counts"], k, seed=seed, workload_id=w["wid"])
        self.choices = d(synth.choices_array(choices, K))
        self.N = len(choices)
        self.T = T = self.N + 1
        self.p_max = T
        self.root = d(synth.root_token_input(w, seed=seed))
        self.plen = d(synth.prefix_lengths(w, seed=seed))
        self.tree = {n: torch.empty(s, dtype=dt, device=dev) for n, s, dt in [
            ("tree_candidates", (B, T), torch.int32), ("tree_indices", (T,), torch.int32),
            ("parent", (T,), torch.int32), ("depth", (T,), torch.int32),
            ("position_ids", (B, T), torch.int32), ("tree_mask", (T, T), torch.uint8),
            ("retrieve", (T, K + 1), torch.int32), ("num_paths", (1,), torch.int32),
            ("status", (2,), torch.int32)]}

        # one heads pass and the tree build (once per tree spec, as the
        # pages build the tree buffers once per medusa_choices); the planted
        # logits need this step's candidates
        self.run_heads()
        self.run_build_tree()
        torch.cuda.synchronize()
        assert self.tree["status"].cpu().tolist() == [0, -1]
        cand = self.tree["tree_candidates"].cpu().numpy()
        ret = self.tree["retrieve"].cpu().numpy()
        npaths = int(self.tree["num_paths"].cpu()[0])
        depth = self.tree["depth"].cpu().numpy()
        self.num_paths_host = npaths

        Hq, dh, S, nl = w["Hq"], w["d"], w["S_max"], w["n_layers"]
        att = synth.attention_inputs(w, depth, synth.prefix_lengths(w, seed=seed), seed=seed)
        self.q = d(att["q"])
        del att
        kc, vc = synth.kv_cache(dict(w, Hkv=Hq), seed=seed)
        self.k_cache, self.v_cache = d(kc), d(vc)
        del kc, vc
        self.layer_elems = B * Hq * S * dh
        self.att_out = torch.empty((B, T, Hq, dh), dtype=torch.bfloat16, device=dev)
        self.att_ws = torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, B, T, Hq, dh, S),
                                  dtype=torch.uint8, device=dev)

        # the acceptance test reads one of NLOGITS logits sets per step, each
        # with its own planted path (accepted lengths vary from step to
        # step), 8.19 MB each: 524 MB in all, so a step's logits never sit in
        # the 256 MB last-level cache
        self.logit_sets = []
        self.plans = []
        for i in range(self.NLOGITS):
            logits, plan = synth.posterior_logits(w, cand, ret, npaths, depth, seed=seed + 7919 * i)
            self.logit_sets.append(d(logits))
            self.plans.append(plan)
            del logits
        self.plan = self.plans[0]
        self.logits = self.logit_sets[0]
        self.logit_index = 0
        self.post = {n: torch.empty(B, dtype=torch.int32, device=dev)
                     for n in ("best_path", "accept_len", "next_token")}
        self.post_ws = torch.zeros(md.medusa_posterior_workspace(B, T, V), dtype=torch.uint8, device=dev)
        self.new_plen = torch.empty(B, dtype=torch.int32, device=dev)
        self.scale = 1.0 / math.sqrt(dh)
        self.layer = 0

    # each stage calls the C entry point directly with pre-marshalled pointers
    def run_resblock(self):
        w, L = self.w, self.md.lib
        rc = L.medusa_resblock(self.md.MEDUSA_BF16, w["B"], w["H"], w["K"], self.hidden.data_ptr(),
                               self.w1.data_ptr(), self.b1.data_ptr(), self.r.data_ptr(), self.stream)
        assert rc == 0, rc

    def run_lm(self):
        """The lm_head + top-k with this step's tree gather in its tail
        (medusa_lm_head_topk_tree: one kernel at this shape)."""
        w, L, t = self.w, self.md.lib, self.tree
        rc = L.medusa_lm_head_topk_tree(self.md.MEDUSA_BF16, w["B"], w["H"], w["V"], w["K"], w["topk"],
                                        self.r.data_ptr(), self.w_lm.data_ptr(), self.topk_ids.data_ptr(),
                                        self.topk_vals.data_ptr(), None, self.T, t["tree_indices"].data_ptr(),
                                        t["depth"].data_ptr(), self.root.data_ptr(), self.plen.data_ptr(),
                                        t["tree_candidates"].data_ptr(), t["position_ids"].data_ptr(),
                                        self.heads_ws.data_ptr(), self.heads_ws.numel(), self.stream)
        assert rc == 0, rc

    def run_heads(self):
        self.run_resblock()
        self.run_lm()

    def run_tree(self):
        """The per-step half of the tree as a launch of its own: this step's
        top-k, root tokens and prefix lengths gathered through the tree built
        at setup (the step itself gathers inside run_lm)."""
        w, L, t = self.w, self.md.lib, self.tree
        rc = L.medusa_tree_candidates(w["B"], self.T, w["K"], w["topk"], t["tree_indices"].data_ptr(),
                                      t["depth"].data_ptr(), self.topk_ids.data_ptr(), self.root.data_ptr(),
                                      self.plen.data_ptr(), t["tree_candidates"].data_ptr(),
                                      t["position_ids"].data_ptr(), self.stream)
        assert rc == 0, rc

    def run_build_tree(self):
        w, L, t = self.w, self.md.lib, self.tree
        rc = L.medusa_build_tree(w["B"], w["K"], w["topk"], self.N, self.choices.data_ptr(),
                                 self.topk_ids.data_ptr(), self.root.data_ptr(), self.plen.data_ptr(),
                                 t["tree_candidates"].data_ptr(), t["tree_indices"].data_ptr(),
                                 t["parent"].data_ptr(), t["depth"].data_ptr(), t["position_ids"].data_ptr(),
                                 t["tree_mask"].data_ptr(), t["retrieve"].data_ptr(), t["num_paths"].data_ptr(),
                                 self.p_max, t["status"].data_ptr(), self.stream)
        assert rc == 0, rc

    def run_attention(self):
        w, L = self.w, self.md.lib
        off = self.layer * self.layer_elems * 2
        rc = L.medusa_tree_attention(self.md.MEDUSA_BF16, w["B"], self.T, w["Hq"], w["d"], w["S_max"],
                                     self.q.data_ptr(), self.k_cache.data_ptr() + off,
                                     self.v_cache.data_ptr() + off, self.plen.data_ptr(),
                                     self.tree["tree_mask"].data_ptr(), self.scale, self.att_out.data_ptr(),
                                     self.att_ws.data_ptr(), self.att_ws.numel(), self.stream)
        assert rc == 0, rc
        self.layer = (self.layer + 1) % w["n_layers"]

    def run_posterior(self):
        w, L, t, p = self.w, self.md.lib, self.tree, self.post
        self.logits = self.logit_sets[self.logit_index]
        self.logit_index = (self.logit_index + 1) % self.NLOGITS
        rc = L.medusa_evaluate_posterior(w["B"], self.T, w["V"], self.p_max, w["K"] + 1, self.logits.data_ptr(),
                                         t["tree_candidates"].data_ptr(), t["retrieve"].data_ptr(),
                                         t["num_paths"].data_ptr(), w["temperature"], w["eps"], w["delta"],
                                         p["best_path"].data_ptr(), p["accept_len"].data_ptr(),
                                         p["next_token"].data_ptr(), self.post_ws.data_ptr(),
                                         self.post_ws.numel(), self.stream)
        assert rc == 0, rc

    def run_commit(self):
        w, L, t, p = self.w, self.md.lib, self.tree, self.post
        rc = L.medusa_commit_kv(self.md.MEDUSA_BF16, w["B"], w["n_layers"], w["Hq"], w["d"], w["S_max"],
                                self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.plen.data_ptr(),
                                t["retrieve"].data_ptr(), self.p_max, w["K"] + 1, p["best_path"].data_ptr(),
                                p["accept_len"].data_ptr(), self.new_plen.data_ptr(), self.stream)
        assert rc == 0, rc

    STAGES = ("resblock", "lm_head_topk_tree", "tree_attention", "posterior", "commit_kv")

    def run(self, events=None, lm_events=None):
        """One verify step.  events: one per stage boundary (breakdown pass);
        lm_events: a pair bracketing the lm_head + top-k (+ tree gather) call
        (timed pass)."""
        fns = (self.run_resblock, self.run_lm, self.run_attention, self.run_posterior, self.run_commit)
        for i, fn in enumerate(fns):
            if events is not None:
                events[i].record()
            if lm_events is not None and i == 1:
                lm_events[0].record()
            fn()
            if lm_events is not None and i == 1:
                lm_events[1].record()
        if events is not None:
            events[len(fns)].record()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "lm_head_topk_vicuna7b_pmc_traffic.md")
HEADS_SOURCE = os.path.join(ROOT, "speculative_decoding_medusa_amd", "csrc", "heads.hip")


def measured_traffic():
    """HBM bytes per lm_head + top-k call from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when that
    summary is missing or was taken on a different heads.hip."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = open(HEADS_SOURCE, "rb").read()
    except OSError:
        return None
    fields = dict(re.findall(r"^(\w+): (\S+)$", text, re.M))
    if fields.get("heads_hip_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return int(float(fields["traffic_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def lm_bytes(w, T):
    """Algorithmic bytes of one lm_head + top-k launch with the tree gather
    in its tail: every weight once, r once, the top-k ids and logits
    written; the gather reads tree_indices and depth (T each), root token and
    prefix length (B each) and one top-k id per node, and writes the
    candidates and positions ([B][T] each)."""
    B, H, V, K, k = w["B"], w["H"], w["V"], w["K"], w["topk"]
    return K * V * H * 2 + B * K * H * 4 + B * K * k * 8 + (2 * T + 2 * B + 3 * B * T) * 4


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_inputs(w, seed):
    import oracle
    import synth

    x = synth.heads_inputs(w, seed=seed)
    choices = synth.choices_array(
        synth.random_tree_choices(w["depth_counts"], w["topk"], seed=seed, workload_id=w["wid"]), w["K"])
    root = synth.root_token_input(w, seed=seed)
    plen = synth.prefix_lengths(w, seed=seed)
    kc, vc = synth.kv_cache(dict(w, Hkv=w["Hq"]), seed=seed)
    hd = oracle.heads(x["hidden"], x["w1"], x["b1"], x["w_lm"], w["topk"])
    tr = oracle.build_tree(choices, w["K"], w["topk"], hd["topk_ids"], root, plen)
    att = synth.attention_inputs(w, tr["depth"], plen, seed=seed)
    logits, _ = synth.posterior_logits(w, tr["tree_candidates"], tr["retrieve"], tr["num_paths"], tr["depth"],
                                       seed=seed)
    return dict(x=x, choices=choices, root=root, plen=plen, kc=kc, vc=vc, att=att, logits=logits)


def _oracle_steps(w, inp, min_steps, min_seconds, max_steps):
    """Whole oracle verify steps, timed until at least ``min_seconds`` of
    oracle work (and ``min_steps`` steps) have run; the median step."""
    import oracle

    x, choices, root, plen, kc, vc = (inp[k] for k in ("x", "choices", "root", "plen", "kc", "vc"))
    att, logits = inp["att"], inp["logits"]
    runs = []
    spent = 0.0
    while len(runs) < max_steps and (len(runs) < min_steps or spent < min_seconds):
        times = {}
        t0 = time.perf_counter()
        hd = oracle.heads(x["hidden"], x["w1"], x["b1"], x["w_lm"], w["topk"])
        t1 = time.perf_counter()
        tr = oracle.build_tree(choices, w["K"], w["topk"], hd["topk_ids"], root, plen)
        t2 = time.perf_counter()
        times["heads"], times["build_tree"] = t1 - t0, t2 - t1
        t2 = time.perf_counter()
        oracle.tree_attention(att["q"], att["k_cache"], att["v_cache"], plen, tr["tree_mask"],
                              1.0 / math.sqrt(w["d"]))
        t3 = time.perf_counter()
        post = oracle.evaluate_posterior(logits, tr["tree_candidates"], tr["retrieve"], tr["num_paths"],
                                         w["temperature"], w["eps"], w["delta"])
        t4 = time.perf_counter()
        oracle.commit_kv(kc, vc, plen, tr["retrieve"], post["best_path"], post["accept_len"])
        t5 = time.perf_counter()
        times["tree_attention"], times["posterior"], times["commit_kv"] = t3 - t2, t4 - t3, t5 - t4
        runs.append(times)
        spent += sum(times.values())
    runs.sort(key=lambda t: sum(t.values()))
    return runs[len(runs) // 2], len(runs), spent


def cpu_baseline(w, seed, min_steps=3, min_seconds=10.0, max_steps=30):
    """The oracle on full steps of the same workload on this host, twice: with
    every core NumPy's thread pools use, and with one thread pinned to the
    first core of this process's affinity set.  Inputs are generated outside
    the timing; each run reports the median step."""
    from threadpoolctl import threadpool_info, threadpool_limits

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    inp = _oracle_inputs(w, seed)
    med, n, spent = _oracle_steps(w, inp, min_steps, min_seconds, max_steps)
    total = sum(med.values())
    cpus = sorted(os.sched_getaffinity(0))
    single = None
    try:
        os.sched_setaffinity(0, {cpus[0]})
        with threadpool_limits(limits=1):
            smed, sn, sspent = _oracle_steps(w, inp, 2, min_seconds, max_steps)
        stotal = sum(smed.values())
        single = {"value": round(1.0 / stotal, 4), "unit": "steps/s", "cores": 1, "pinned_cpu": cpus[0],
                  "seconds_per_step": round(stotal, 3), "stage_seconds": {k: round(v, 3) for k, v in smed.items()},
                  "sample": "median of %d full verify steps (%.1f s)" % (sn, sspent)}
    finally:
        os.sched_setaffinity(0, set(cpus))
    return {"value": round(1.0 / total, 4), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": "median of %d full verify steps (%.1f s of oracle work) at the same shapes "
                      "(5 heads, 64-node tree, one attention layer at prefix 2048, typical posterior over "
                      "64x32000, 32-layer commit), fp64 NumPy, all cores" % (n, spent),
            "seconds_per_step": round(total, 3), "stage_seconds": {k: round(v, 3) for k, v in med.items()},
            "single_thread": single, "nproc": os.cpu_count(), "affinity_cpus": len(cpus),
            "cpu_model": _cpu_model()}


def graph_timing(step, steps):
    """The same verify step replayed from HIP graphs: each graph captures
    `per` consecutive steps (their attention layers in order, so the graphs
    together cover the rotating 32-layer cache), captured on a side stream
    of default priority, then exactly `steps` steps replayed in layer order,
    bracketed by events on the stream they run on.  Several steps per graph
    spread the graph launch (about 4 us) over them: one step per graph ran
    at 3,756 steps/s, four at 3,806, eight at 3,815 and 32 at 3,820 against
    3,818 eager (one process)."""
    import torch
    n = step.w["n_layers"]
    per = next(p for p in (8, 4, 2, 1) if n % p == 0 and steps % p == 0)
    saved_stream, saved_layer = step.stream, step.layer
    side = torch.cuda.Stream()
    graphs = []
    torch.cuda.synchronize()
    for layer in range(0, n, per):
        g = torch.cuda.CUDAGraph()
        step.layer = layer
        with torch.cuda.graph(g, stream=side):
            step.stream = torch.cuda.current_stream().cuda_stream
            for _ in range(per):
                step.run()
        graphs.append(g)
    step.stream, step.layer = saved_stream, saved_layer
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps // per):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return {"value": round(1000.0 / ms, 2), "unit": "steps/s", "ms_per_step": round(ms, 4), "graphs": len(graphs),
            "steps_per_graph": per,
            "note": "the whole step replayed from HIP graphs (%d graphs of %d consecutive steps, one attention "
                    "layer each), %d steps" % (len(graphs), per, steps)}


def base_head_timing(step, seed, steps):
    """The base model's lm_head over the 64 tree nodes (packed bf16 weights,
    H x V of the workload): the step that produces the acceptance test's
    logits, outside the verify step's own metric.  Two weight copies (the
    second the negated first) alternate so the stream never sits in the last-
    level cache; `steps` calls timed with events on the stream they run on.
    Also timed: the acceptance test on those logits, unfused (lm_head, then
    medusa_evaluate_posterior) and fused (medusa_base_posterior: row
    statistics in the lm_head's epilogue, the logits never written)."""
    import numpy as np
    import torch

    import speculative_decoding_medusa_amd as md
    import synth
    w = step.w
    dev = torch.device("cuda:0")
    T, H, V = step.T, w["H"], w["V"]
    x = synth.base_head_inputs(T, H, V, seed=seed)
    hidden = torch.from_numpy(x["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    wb = torch.from_numpy(x["w_base"].view(np.int16)).to(dev).view(torch.bfloat16)
    packs = [md.medusa_base_lm_head_pack(wb), md.medusa_base_lm_head_pack(wb.neg())]
    del wb
    out = torch.empty((1, T, V), dtype=torch.float32, device=dev)
    h3 = hidden.view(1, T, H)
    tr = step.tree
    post = {n: torch.empty(1, dtype=torch.int32, device=dev) for n in ("best_path", "accept_len", "next_token")}
    ws_p = torch.zeros(md.medusa_posterior_workspace(1, T, V), dtype=torch.uint8, device=dev)
    ws_f = torch.zeros(md.medusa_base_posterior_workspace(1, T, H, V), dtype=torch.uint8, device=dev)
    temp, eps, delta = w["temperature"], w["eps"], w["delta"]

    # every call through the C entry points with pre-marshalled pointers (as
    # the verify step's stages), so the host's per-call cost in the binding
    # cannot leave the GPU idle between calls
    L, sp = md.lib, torch.cuda.current_stream().cuda_stream
    p_max, D = tr["retrieve"].shape
    hp, op = h3.data_ptr(), out.data_ptr()
    pp = [pk.data_ptr() for pk in packs]
    cand, ret, npth = tr["tree_candidates"].data_ptr(), tr["retrieve"].data_ptr(), tr["num_paths"].data_ptr()
    bp, ap, np_ = post["best_path"].data_ptr(), post["accept_len"].data_ptr(), post["next_token"].data_ptr()

    def gemm(i):
        assert L.medusa_base_lm_head(md.MEDUSA_BF16, T, H, V, hp, pp[i % 2], 1, op, sp) == 0

    def unfused(i):
        gemm(i)
        assert L.medusa_evaluate_posterior(1, T, V, p_max, D, op, cand, ret, npth, temp, eps, delta, bp, ap, np_,
                                           ws_p.data_ptr(), ws_p.numel(), sp) == 0

    def fused(i):
        assert L.medusa_base_posterior(1, T, H, V, p_max, D, hp, pp[i % 2], 1, cand, ret, npth, temp, eps, delta,
                                       bp, ap, np_, ws_f.data_ptr(), ws_f.numel(), sp) == 0

    def timed(fn):
        # for the first ~10 ms after the weights are packed the GEMM runs
        # about 10% slower (53 against 48 us per call, then steady in every
        # later batch); warm up past that and time the steady state
        for i in range(300):
            fn(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1000.0 / steps

    us = timed(gemm)
    us_unfused = timed(unfused)
    us_fused = timed(fused)
    nbytes = V * H * 2 + T * H * 2 + T * V * 4
    gbs = nbytes / us / 1e3
    return {"kernel": "base_lm_head", "M": T, "H": H, "V": V, "layout": "packed", "mean_launch_us": round(us, 2),
            "bound": "hbm", "bytes_per_launch": nbytes, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_tflops": round(2.0 * T * H * V / us / 1e6, 1),
            "with_acceptance_us": {"unfused": round(us_unfused, 2), "fused": round(us_fused, 2),
                                   "temperature": temp}}


def copy_peak_gbs(nbytes=1 << 30, n=20):
    """A measured streaming-copy rate for the roofline: a device-to-device
    copy of nbytes (nbytes read + nbytes written per call), GB/s by HIP
    events over n calls."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    us = _time_calls(lambda i: dst.copy_(src), n)
    del src, dst
    return 2.0 * nbytes / (us * 1e-6) / 1e9


def _time_calls(fn, n, warm=3):
    """Mean microseconds per call of fn(i) over n calls, HIP events on the
    current stream (where the library enqueues)."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1000.0 / n


def _attention_caller(md, q, kcs, vcs, plen, mask, out, ws):
    """fn(i): one medusa_tree_attention call on layer i % len(kcs), through
    the C entry point with pre-marshalled pointers (no binding overhead
    between the timed calls)."""
    import torch
    B, T, Hq, d = q.shape
    S = kcs[0].shape[2]
    sp = torch.cuda.current_stream().cuda_stream
    kp, vp = [k.data_ptr() for k in kcs], [v.data_ptr() for v in vcs]
    args = (q.data_ptr(), plen.data_ptr(), mask.data_ptr(), float(d) ** -0.5, out.data_ptr(), ws.data_ptr(),
            ws.numel())

    def fn(i):
        j = i % len(kp)
        assert md.lib.medusa_tree_attention(md.MEDUSA_BF16, B, T, Hq, d, S, args[0], kp[j], vp[j], args[1], args[2],
                                            args[3], args[4], args[5], args[6], sp) == 0
    return fn


def nucleus_timing(step, seed, steps):
    """Nucleus (top-p 0.8, temperature 0.7) acceptance over the step's
    [64][32000] logits and tree: the whole call (one draw per node, then the
    decision), HIP events around the calls.  The sampling kernel reads the
    logits in its passes from LDS or registers, so its HBM floor is one read
    of T x V x 4 bytes."""
    import torch

    import speculative_decoding_medusa_amd as md
    import synth
    w = step.w
    t = step.tree
    B, T, V = w["B"], step.T, w["V"]
    u = torch.from_numpy(synth.node_uniforms(w, T, seed=seed)).to(step.dev)
    out = {n: torch.empty(B, dtype=torch.int32, device=step.dev) for n in ("best_path", "accept_len", "next_token")}
    ws = torch.zeros(md.medusa_posterior_nucleus_workspace(B, T), dtype=torch.uint8, device=step.dev)
    p_max, D = t["retrieve"].shape
    sp = torch.cuda.current_stream().cuda_stream
    ptrs = (step.logits.data_ptr(), t["tree_candidates"].data_ptr(), t["retrieve"].data_ptr(),
            t["num_paths"].data_ptr(), u.data_ptr(), out["best_path"].data_ptr(), out["accept_len"].data_ptr(),
            out["next_token"].data_ptr())

    def call(i):
        assert md.lib.medusa_evaluate_posterior_nucleus(B, T, V, p_max, D, ptrs[0], ptrs[1], ptrs[2], ptrs[3], 0.7,
                                                        0.8, ptrs[4], ptrs[5], ptrs[6], ptrs[7], None,
                                                        ws.data_ptr(), ws.numel(), sp) == 0
    us = _time_calls(call, steps)
    byt = B * T * V * 4
    return {"us": round(us, 2), "top_p": 0.8, "temperature": 0.7, "bytes": byt,
            "achieved": round(byt / us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(byt / us / 1e3 / HBM_PEAK_GBS, 4),
            "note": "latency- and LDS-bound: three radix passes over each node's vocabulary on one workgroup "
                    "per node"}


def sample_typical_timing(step, seed, steps):
    """Typical mode's sampled next token on the step's
    [64][32000] logits, drawn at the root (best path 0, nothing accepted):
    the whole call, HIP events around the calls, the step key advancing per
    call.  One 32000-token row (128 KB) is read once into one workgroup's
    registers, so the call is bound by that compute unit's ALUs, not by
    bandwidth."""
    import torch

    import speculative_decoding_medusa_amd as md
    w = step.w
    t = step.tree
    B, T, V = w["B"], step.T, w["V"]
    p_max, D = t["retrieve"].shape
    best = torch.zeros(B, dtype=torch.int32, device=step.dev)
    acc = torch.zeros(B, dtype=torch.int32, device=step.dev)
    nxt = torch.empty(B, dtype=torch.int32, device=step.dev)
    sp = torch.cuda.current_stream().cuda_stream
    ptrs = (step.logits.data_ptr(), t["retrieve"].data_ptr(), best.data_ptr(), acc.data_ptr(), nxt.data_ptr())

    def call(i):
        assert md.lib.medusa_sample_typical(B, T, V, p_max, D, ptrs[0], ptrs[1], ptrs[2], ptrs[3], w["temperature"],
                                            w["eps"], w["delta"], seed, i, ptrs[4], sp) == 0
    us = _time_calls(call, steps)
    return {"us": round(us, 2), "temperature": w["temperature"], "bytes": B * V * 4,
            "note": "one workgroup per sequence; the row is read once into registers; bound by that "
                    "compute unit's vector ALUs"}


def attention_prefix_sweep(step, steps):
    """Tree attention (64-node tree, 32 heads x 128) at prefixes 512, 1024,
    2048 and 4096, eight layers of KV rotated so no layer sits in the
    last-level cache; algorithmic bytes (every prefix and tree K/V row once,
    Q in, output out) over the mean duration of the call."""
    import torch

    import speculative_decoding_medusa_amd as md
    w = step.w
    dev = torch.device("cuda:0")
    T, Hq, d = step.T, w["Hq"], w["d"]
    gen = torch.Generator(device=dev).manual_seed(3)
    q = (torch.randn((1, T, Hq, d), generator=gen, device=dev)).to(torch.bfloat16)
    out = torch.empty_like(q)
    rows = []
    for L in w["L_sweep"]:
        S = L + T + 8
        nl = 8
        kc = [torch.randn((1, Hq, S, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nl)]
        vc = [torch.randn((1, Hq, S, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nl)]
        plen = torch.full((1,), L, dtype=torch.int32, device=dev)
        ws = torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, 1, T, Hq, d, S), dtype=torch.uint8,
                         device=dev)
        us = _time_calls(_attention_caller(md, q, kc, vc, plen, step.tree["tree_mask"], out, ws), steps)
        nbytes = 2 * Hq * (L + T) * d * 2 + 2 * T * Hq * d * 2
        rows.append({"L": L, "us": round(us, 2), "bytes": nbytes, "achieved": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del kc, vc
    return {"unit": "GB/s", "peak": HBM_PEAK_GBS, "T": T, "Hq": Hq, "d": d, "rows": rows}


def attention_only(args):
    """Tree attention alone at prefix args.attention: the Vicuna-7B layer
    (64-node tree of the bench's spec, 32 heads x 128, bf16), eight layers of
    KV rotated, args.steps calls timed with events on the library's stream."""
    import numpy as np
    import torch

    import speculative_decoding_medusa_amd as md
    import synth
    w = synth.workload("vicuna-7b")
    dev = torch.device("cuda:0")
    choices = synth.random_tree_choices(w["depth_counts"], w["topk"], seed=args.seed, workload_id=w["wid"])
    T, Hq, d, L = len(choices) + 1, w["Hq"], w["d"], args.attention
    ids = torch.zeros((1, w["K"], w["topk"]), dtype=torch.int32, device=dev)
    tree = md.medusa_build_tree(torch.from_numpy(synth.choices_array(choices, w["K"])).to(dev), ids,
                                torch.zeros(1, dtype=torch.int32, device=dev),
                                torch.full((1,), L, dtype=torch.int32, device=dev))
    gen = torch.Generator(device=dev).manual_seed(3)
    q = torch.randn((1, T, Hq, d), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    S, nl = L + T, 8
    kc = [torch.randn((1, Hq, S, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nl)]
    vc = [torch.randn((1, Hq, S, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nl)]
    plen = torch.full((1,), L, dtype=torch.int32, device=dev)
    ws = torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, 1, T, Hq, d, S), dtype=torch.uint8,
                     device=dev)
    us = _time_calls(_attention_caller(md, q, kc, vc, plen, tree["tree_mask"], out, ws), args.steps)
    nbytes = 2 * Hq * (L + T) * d * 2 + 2 * T * Hq * d * 2
    print(json.dumps({"attention": {"L": L, "T": T, "Hq": Hq, "d": d, "max_slots": S, "calls": args.steps,
                                    "us": round(us, 2), "bytes": nbytes, "achieved": round(nbytes / us / 1e3, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s"}}))


def batch8_33b(step, seed, steps):
    """The whole verify step at the Vicuna-33B batch-8 shape (packed heads)."""
    return whole_step(step, "vicuna-33b-b8", seed, steps, packed=True)


def vicuna13b(step, seed, steps):
    """The whole verify step at the Vicuna-13B shape, batch 1 (row-major heads)."""
    return whole_step(step, "vicuna-13b", seed, steps, packed=False)


def whole_step(step, wname, seed, steps, packed):
    """A whole verify step at a named workload's shape: the heads (5 heads,
    top-10; packed: W1 and lm_head packed once and medusa_heads_packed, the
    row-major calls timed beside it; else the row-major calls, the packed
    ones timed beside them), the per-step tree gather on the 64-node tree of
    the 7B step, one tree attention layer (two layers of KV rotated), typical
    acceptance (T 0.7) over [B][64][32000] logits and the commit across every
    layer of the cache.  Random device data (timing only; the layers
    attention does not read are left uninitialised).  Each stage timed alone
    with HIP events, then the chained step; algorithmic bytes over the mean
    duration of each call."""
    import numpy as np
    import torch

    import speculative_decoding_medusa_amd as md
    import synth
    w = synth.workload(wname)
    dev = torch.device("cuda:0")
    B, H, V, K, k, Hq, d = w["B"], w["H"], w["V"], w["K"], w["topk"], w["Hq"], w["d"]
    n_layers = w["n_layers"]
    gen = torch.Generator(device=dev).manual_seed(seed + 7)
    bf, i32 = torch.bfloat16, torch.int32
    hidden = torch.randn((B, H), generator=gen, device=dev).to(bf)
    w1 = (torch.randn((K, H, H), generator=gen, device=dev) * 0.02).to(bf)
    b1 = (torch.randn((K, H), generator=gen, device=dev) * 0.02).to(bf)
    w_lm = torch.empty((K, V, H), dtype=bf, device=dev)
    for h in range(K):
        w_lm[h] = (torch.randn((V, H), generator=gen, device=dev) * 0.02).to(bf)
    ws = torch.zeros(md.medusa_heads_workspace(md.MEDUSA_BF16, B, H, V, K, k), dtype=torch.uint8, device=dev)
    r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
    topk = dict(topk_ids=torch.empty((B, K, k), dtype=i32, device=dev),
                topk_logits=torch.empty((B, K, k), dtype=torch.float32, device=dev))
    w_packed = md.medusa_heads_pack(w_lm)
    w1_packed = md.medusa_heads_pack(w1)
    nrep = max(10, steps // 4)

    def heads_packed(i):
        md.medusa_heads_packed(hidden, w1_packed, b1, w_packed, V, k, out=topk, ws=ws)

    def heads_row_major(i):
        md.medusa_resblock(hidden, w1, b1, r=r)
        md.medusa_lm_head_topk(r, w_lm, k, out=topk, ws=ws)

    heads, other = (heads_packed, heads_row_major) if packed else (heads_row_major, heads_packed)
    us_heads_other = _time_calls(other, nrep)
    heads_bytes = K * (H * H + H * V + H) * 2 + B * H * 2

    # the tree (built once from the 7B step's spec) and its per-step gather
    T = step.T
    plen_host = np.asarray(synth.prefix_lengths(w, seed=seed), dtype=np.int32)
    S = max(int(plen_host.max()) + T + 8, w["S_max"])
    plen = torch.from_numpy(plen_host).to(dev)
    root = torch.randint(0, V, (B,), generator=gen, device=dev, dtype=i32)
    heads(0)
    tree = md.medusa_build_tree(step.choices, topk["topk_ids"], root, plen, p_max=T)
    torch.cuda.synchronize()
    assert tree["status"].cpu().tolist() == [0, -1]

    def gather(i):
        md.medusa_tree_candidates(tree["tree_indices"], tree["depth"], topk["topk_ids"], root, plen, out=tree)

    # 60-layer caches; attention rotates over two initialised layers
    kc = torch.empty((n_layers, B, Hq, S, d), dtype=bf, device=dev)
    vc = torch.empty_like(kc)
    for layer in range(2):
        kc[layer].normal_(generator=gen)
        vc[layer].normal_(generator=gen)
    q = torch.randn((B, T, Hq, d), generator=gen, device=dev).to(bf)
    att = torch.empty_like(q)
    aws = torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, B, T, Hq, d, S), dtype=torch.uint8,
                      device=dev)

    def attention(i):
        md.medusa_tree_attention(q, kc[i % 2], vc[i % 2], plen, tree["tree_mask"], d ** -0.5, out=att, ws=aws)

    logits = torch.randn((B, T, V), generator=gen, device=dev) * w["logit_std"]
    post = {n: torch.empty(B, dtype=i32, device=dev) for n in ("best_path", "accept_len", "next_token")}
    pws = torch.zeros(md.medusa_posterior_workspace(B, T, V), dtype=torch.uint8, device=dev)

    def posterior(i):
        md.medusa_evaluate_posterior(logits, tree["tree_candidates"], tree["retrieve"], tree["num_paths"],
                                     w["temperature"], w["eps"], w["delta"], out=post, ws=pws)

    new_plen = torch.empty(B, dtype=i32, device=dev)

    def commit(i):
        md.medusa_commit_kv(kc, vc, plen, tree["retrieve"], post["best_path"], post["accept_len"],
                            new_prefix_len=new_plen)

    def whole(i):
        heads(i)
        gather(i)
        attention(i)
        posterior(i)
        commit(i)

    us = {name: _time_calls(fn, nrep) for name, fn in (("heads", heads), ("tree_candidates", gather),
                                                        ("tree_attention", attention), ("posterior", posterior),
                                                        ("commit_kv", commit))}
    us_step = _time_calls(whole, nrep)
    att_bytes = int(sum(2 * Hq * (int(L) + T) * d * 2 for L in plen_host)) + B * 2 * T * Hq * d * 2
    del w1, w_lm, w_packed, w1_packed, kc, vc
    label = "%s verify step, batch %d" % (wname.split("-b")[0] if wname.endswith("-b8") else wname, B)
    return {"workload": label, "B": B, "H": H, "V": V, "K": K, "topk": k, "Hq": Hq,
            "d": d, "T": T, "n_layers": n_layers, "prefix_lens": plen_host.tolist(), "unit": "GB/s",
            "peak": HBM_PEAK_GBS,
            "steps_per_s": round(1e6 / us_step, 2), "step_us": round(us_step, 2),
            "stages_us": {n: round(v, 2) for n, v in us.items()},
            "heads": {"us": round(us["heads"], 2), "bytes": heads_bytes,
                      "achieved": round(heads_bytes / us["heads"] / 1e3, 1),
                      "frac": round(heads_bytes / us["heads"] / 1e3 / HBM_PEAK_GBS, 4),
                      "weights": "packed" if packed else "row-major",
                      ("us_row_major_weights" if packed else "us_packed_weights"): round(us_heads_other, 2)},
            "tree_attention": {"us": round(us["tree_attention"], 2), "bytes": att_bytes,
                               "achieved": round(att_bytes / us["tree_attention"] / 1e3, 1),
                               "frac": round(att_bytes / us["tree_attention"] / 1e3 / HBM_PEAK_GBS, 4)},
            "note": "each stage timed alone over %d calls, then the chained step over %d; HIP events on the "
                    "library's stream (a stage of one small kernel timed alone is bound by the host's launch "
                    "rate through the Python binding)" % (nrep, nrep)}


SWEEP_K = (3, 4, 5, 8)
SWEEP_T = (16, 32, 64, 128)


def tree_sweep(args):
    """Cost of one verify step against the tree's shape (Vicuna-7B sizes,
    batch 1): for each number of heads K and tree size T, the T - 1 rank
    tuples with the highest acceptance probability under the synthetic
    acceptance model (synth.geometric_acceptance) form the tree; a step
    (K heads, tree, one attention layer at prefix L, acceptance on T x V
    logits, commit over every layer) is captured in a HIP graph and its
    replays timed with events on the capture stream, and the heads alone
    likewise.  Reported beside it: the model's expected tokens per step
    (accepted length + the bonus token) and their ratio to the step time.
    Weights and activations are random on the device (timing does not
    depend on their values)."""
    import torch

    import speculative_decoding_medusa_amd as md
    import synth

    w = synth.workload("vicuna-7b")
    dev = torch.device("cuda:0")
    B, H, V, k = 1, w["H"], w["V"], w["topk"]
    Hq, dh, L, nl = w["Hq"], w["d"], w["L"], w["n_layers"]
    Kmax, Tmax = max(SWEEP_K), max(SWEEP_T)
    S = L + Tmax + 8
    bf = torch.bfloat16
    gen = torch.Generator(device=dev).manual_seed(args.seed)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device=dev) * std).to(bf)

    hidden = rnd((B, H), 1.0)
    w1, b1 = rnd((Kmax, H, H), 0.02), rnd((Kmax, H), 0.02)
    w_lm = torch.empty((Kmax, V, H), dtype=bf, device=dev)
    for h in range(Kmax):
        w_lm[h] = rnd((V, H), 0.02)
    kc = torch.empty((nl, B, Hq, S, dh), dtype=bf, device=dev)
    vc = torch.empty_like(kc)
    for layer in range(nl):
        kc[layer] = rnd((B, Hq, S, dh), 1.0)
        vc[layer] = rnd((B, Hq, S, dh), 1.0)
    plen = torch.full((B,), L, dtype=torch.int32, device=dev)
    root = torch.full((B,), 7, dtype=torch.int32, device=dev)
    i32 = torch.int32

    def time_graph(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1000.0 / args.steps

    rows = []
    for K in SWEEP_K:
        acc_model = synth.geometric_acceptance(K, k)
        r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
        heads = dict(topk_ids=torch.empty((B, K, k), dtype=i32, device=dev),
                     topk_logits=torch.empty((B, K, k), dtype=torch.float32, device=dev))
        ws_h = torch.zeros(md.medusa_heads_workspace(md.MEDUSA_BF16, B, H, V, K, k), dtype=torch.uint8,
                           device=dev)
        w1k, b1k, wlk = w1[:K], b1[:K], w_lm[:K]

        def run_heads():
            md.medusa_resblock(hidden, w1k, b1k, r=r)
            md.medusa_lm_head_topk(r, wlk, k, out=heads, ws=ws_h)

        heads_us = time_graph(run_heads)
        for T in SWEEP_T:
            choices = synth.best_tree_choices(acc_model, T - 1)
            expect = synth.expected_accept_length(acc_model, choices)
            ch = torch.from_numpy(synth.choices_array(choices, K)).to(dev)
            tree = dict(tree_candidates=torch.empty((B, T), dtype=i32, device=dev),
                        tree_indices=torch.empty(T, dtype=i32, device=dev),
                        parent=torch.empty(T, dtype=i32, device=dev), depth=torch.empty(T, dtype=i32, device=dev),
                        position_ids=torch.empty((B, T), dtype=i32, device=dev),
                        tree_mask=torch.empty((T, T), dtype=torch.uint8, device=dev),
                        retrieve=torch.empty((T, K + 1), dtype=i32, device=dev),
                        num_paths=torch.empty(1, dtype=i32, device=dev), status=torch.empty(2, dtype=i32, device=dev))
            q = rnd((B, T, Hq, dh), 1.0)
            att = torch.empty_like(q)
            ws_a = torch.zeros(md.medusa_tree_attention_workspace(md.MEDUSA_BF16, B, T, Hq, dh, S),
                               dtype=torch.uint8, device=dev)
            logits = torch.randn((B, T, V), generator=gen, device=dev) * w["logit_std"]
            post = {n: torch.empty(B, dtype=i32, device=dev) for n in ("best_path", "accept_len", "next_token")}
            ws_p = torch.zeros(md.medusa_posterior_workspace(B, T, V), dtype=torch.uint8, device=dev)
            new_plen = torch.empty(B, dtype=i32, device=dev)

            run_heads()
            md.medusa_build_tree(ch, heads["topk_ids"], root, plen, p_max=T, out=tree)   # once per tree

            def run_step():
                run_heads()
                md.medusa_tree_candidates(tree["tree_indices"], tree["depth"], heads["topk_ids"], root, plen,
                                          out=tree)
                md.medusa_tree_attention(q, kc[0], vc[0], plen, tree["tree_mask"], dh ** -0.5, out=att, ws=ws_a)
                md.medusa_evaluate_posterior(logits, tree["tree_candidates"], tree["retrieve"], tree["num_paths"],
                                             w["temperature"], w["eps"], w["delta"], out=post, ws=ws_p)
                md.medusa_commit_kv(kc, vc, plen, tree["retrieve"], post["best_path"], post["accept_len"],
                                    new_prefix_len=new_plen)

            us = time_graph(run_step)
            status = tree["status"].cpu().tolist()
            if status != [0, -1]:
                raise RuntimeError("tree build failed for K=%d T=%d: %s" % (K, T, status))
            tps = 1.0 + expect
            rows.append({"K": K, "topk": k, "T": T, "depth": max(len(t) for t in choices),
                         "us_per_step": round(us, 2), "heads_us": round(heads_us, 2),
                         "rest_us": round(us - heads_us, 2), "expected_tokens_per_step": round(tps, 4),
                         "tokens_per_ms": round(tps / us * 1000.0, 3)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"tree_sweep": rows, "workload": "vicuna-7b verify step, batch 1 (H %d, V %d, L %d, "
                      "%d layers, one attention layer per step)" % (H, V, L, nl),
                      "acceptance_model": "p[d][i] = q1 gamma^d (1 - rho) rho^i, q1 0.85, gamma 0.9, rho 0.5",
                      "steps": args.steps, "timing": "HIP graph replays, events on the capture stream"}))


GEN_CFG = dict(H=1024, heads=16, I=2816, layers=4, V=32000, eps=1e-6, theta=10000.0)


def _fit_heads(hidden_rows, seq, first, K, V, scale=8.0):
    """Heads fitted to a known continuation: ResBlocks zero (r = h) and head
    j's lm_head the minimum-norm linear map from the final hidden state at
    position first + r to `scale` on token seq[first + r + j + 2] (rows past
    the sequence end get no target).  Host setup for the benchmark only."""
    import numpy as np
    n, H = hidden_rows.shape
    G = hidden_rows @ hidden_rows.T + 1e-6 * np.eye(n)
    w = np.zeros((K, V, H))
    for j in range(K):
        Y = np.zeros((n, V))
        for r in range(n):
            t = first + r + j + 2
            if t < len(seq):
                Y[r, seq[t]] = scale
        w[j] = np.linalg.solve(G, Y).T @ hidden_rows
    return w


def generate_bench(args):
    """End-to-end greedy generation on a small LLaMA-style model (GEN_CFG,
    random weights) through the library's forward pieces: plain greedy (one
    base-model forward per token) against Medusa greedy (heads, tree, one
    forward of the tree, acceptance, commit per step) with K = 3 heads and a
    full binary tree of depth 3 (15 nodes).  Heads: random, and fitted on
    the host to the plain run's own continuation (an upper bound on what
    trained heads accept).  Every run's tokens are checked against the plain
    run's.  Each loop also runs with its step captured in a HIP graph and
    replayed (bookkeeping on the device; a Medusa run may overshoot by a few
    steps between the host's checks).  Wall-clock time of whole generate
    calls (median of 3), prefill and graph capture included."""
    import numpy as np
    import torch

    import synth
    from speculative_decoding_medusa_amd.decoder import TinyDecoder

    dev = torch.device("cuda:0")
    cfg = GEN_CFG
    P, n, K, topk = 32, 128, 3, 2
    model = synth.tiny_decoder(cfg, seed=args.seed)
    prompt = [int(t) for t in np.random.default_rng(args.seed).integers(cfg["V"], size=P)]
    dec = TinyDecoder(model, dev, max_slots=P + n + 64)
    choices = torch.from_numpy(synth.choices_array(synth.full_tree_choices(K, topk), K)).to(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            out = fn()
            torch.cuda.synchronize()
            runs.append(time.perf_counter() - t0)
        return out, sorted(runs)[1]

    ref, t_plain = timed(lambda: dec.greedy(prompt, n))
    ref_g, t_plain_g = timed(lambda: dec.greedy_graph(prompt, n))
    # hidden states along the plain continuation, for the fitted heads; the
    # same forward's logits give every step's top-2 gap
    hidden, logits = dec.prefill(prompt + ref[:-1])
    rows = hidden[0, P - 1:P - 1 + n].float().cpu().numpy().astype(np.float64)
    zz = logits[0, P - 1:P - 1 + n].float().cpu().numpy()
    z = np.sort(zz, axis=1)
    gaps = z[:, -1] - z[:, -2]

    # the activations are bf16, so forwards that sum in different orders (one
    # token, a 15-node tree, a prefill) agree on a logit only to about 1e-2,
    # and a continuation can leave another at a near-tie; where one does,
    # the gap between the two tokens (by the prefill, a third summation
    # order) is reported
    def compare(toks):
        diff = [i for i in range(n) if i >= len(toks) or toks[i] != ref[i]]
        out = {"equal_to_plain": toks == ref}
        if diff:
            i = diff[0]
            out["first_difference"] = i
            if i < len(toks):
                out["logit_gap_there"] = round(float(abs(zz[i, ref[i]] - zz[i, toks[i]])), 5)
        return out
    fitted = _fit_heads(rows, prompt + ref, P - 1, K, cfg["V"])

    def to_bf16(a):
        return torch.from_numpy(synth.bf16_bits(np.asarray(a, dtype=np.float32)).view(np.int16)).to(dev).view(
            torch.bfloat16)

    H, V = cfg["H"], cfg["V"]
    rnd = synth.tiny_heads(cfg, K, seed=args.seed + 1)
    head_sets = {
        "random_heads": {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(dev).view(torch.bfloat16)
                         for k, v in rnd.items()},
        "fitted_heads": dict(w1=torch.zeros((K, H, H), dtype=torch.bfloat16, device=dev),
                             b1=torch.zeros((K, H), dtype=torch.bfloat16, device=dev),
                             w_lm=to_bf16(fitted.reshape(K, V, H))),
    }
    res = {"plain": {"tokens_per_s": round(n / t_plain, 1), "ms": round(t_plain * 1e3, 2), "forwards": n},
           "plain_graph": dict({"tokens_per_s": round(n / t_plain_g, 1), "ms": round(t_plain_g * 1e3, 2)},
                               **compare(ref_g))}
    def histogram(accepts):
        h = [0] * (K + 1)
        for a in accepts:
            h[a] += 1
        return h

    for name, heads in head_sets.items():
        (toks, accepts, _), t = timed(lambda: dec.medusa(heads, choices, topk, prompt, n))
        res["medusa_" + name] = dict({"tokens_per_s": round(n / t, 1), "ms": round(t * 1e3, 2),
                                      "steps": len(accepts), "tokens_per_step": round(n / len(accepts), 3),
                                      "accept_len_histogram": histogram(accepts),
                                      "speedup_vs_plain": round(t_plain / t, 3)}, **compare(toks))
        (toks, steps), t = timed(lambda: dec.medusa_graph(heads, choices, topk, prompt, n))
        res["medusa_" + name + "_graph"] = dict({"tokens_per_s": round(n / t, 1), "ms": round(t * 1e3, 2),
                                                 "steps_run": steps,
                                                 "speedup_vs_plain_graph": round(t_plain_g / t, 3)},
                                                **compare(toks))
    # sampled modes (temperature 0.7): plain sampling one token per forward,
    # and Medusa with typical acceptance and a drawn bonus token, fitted heads
    samp = dict(temperature=0.7, eps=0.09, delta=0.3, seed=args.seed + 5)
    st, t_ps = timed(lambda: dec.sample(prompt, n, mode="typical", **samp))
    res["plain_sampled_typical"] = {"tokens_per_s": round(n / t_ps, 1), "ms": round(t_ps * 1e3, 2)}
    heads = head_sets["fitted_heads"]
    (toks, accepts), t = timed(lambda: dec.medusa_sampled(heads, choices, topk, prompt, n, mode="typical", **samp))
    res["medusa_sampled_typical_fitted_heads"] = {
        "tokens_per_s": round(n / t, 1), "ms": round(t * 1e3, 2), "steps": len(accepts),
        "tokens_per_step": round(n / len(accepts), 3), "accept_len_histogram": histogram(accepts),
        "speedup_vs_plain_sampled": round(t_ps / t, 3),
        "note": "heads fitted to the greedy continuation; sampled continuations leave it, so fewer are accepted"}
    print(json.dumps({"generate": res, "plain_top2_gap": {"smallest": round(float(gaps.min()), 5),
                                                         "at_step": int(np.argmin(gaps)),
                                                         "median": round(float(np.median(gaps)), 5)},
                      "model": dict(cfg), "prompt_len": P, "new_tokens": n, "K": K,
                      "tree": "full binary, depth 3 (15 nodes)", "timing": "wall clock of whole generate calls, "
                      "median of 3, after one warm-up call", "data": "synthetic random weights"}))


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py: this build runs the verify step on one GPU only; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.tree_sweep:
        tree_sweep(args)
        return
    if args.attention:
        attention_only(args)
        return
    if args.generate:
        generate_bench(args)
        return

    import torch

    import synth

    w = synth.workload("vicuna-7b")
    step = Step(w, args.seed)
    nst = len(Step.STAGES)

    # settle: after the seconds of host-side setup the GPU has been idle, and
    # for its first ~10 ms of load it runs the step about 3% slower (20 steps
    # after 5 warm-up steps: 3,614-3,624 steps/s; after 200: 3,719).  Steps
    # run untimed until SETTLE_MS of GPU time have passed, then the W warm-up
    # steps, then the K timed ones.
    settle_steps = 0
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    while True:
        for _ in range(10):
            step.run()
        settle_steps += 10
        t1.record()
        t1.synchronize()
        if t0.elapsed_time(t1) >= SETTLE_MS:
            break
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # timed region: K whole steps; the only events inside bracket the
    # lm_head + top-k call (the roofline kernel), on the stream it runs on,
    # in one step of every LM_SAMPLE: an event record between kernels costs
    # the stream a few microseconds, so bracketing every call would slow the
    # very steps being timed (about 9 us per step measured)
    sampled = list(range(0, args.steps, LM_SAMPLE))
    lm_ev = {s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for s in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step.run(lm_events=lm_ev.get(s))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    lm_ms = [lm_ev[s][0].elapsed_time(lm_ev[s][1]) for s in sampled]

    # per-stage breakdown: a separate, untimed pass of STAGE_STEPS steps with
    # an event at every stage boundary (median, p10 and p90 per stage)
    nb = STAGE_STEPS
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(nb)]
    for s in range(nb):
        step.run(ev[s])
    torch.cuda.synchronize()
    stage_ms = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(nb)] for i in range(nst)]
    # accepted lengths over one pass of the logits sets (untimed)
    hist = [0] * (w["K"] + 1)
    for _ in range(Step.NLOGITS):
        step.run_posterior()
        hist[int(step.post["accept_len"].cpu()[0])] += 1

    def stats(xs):
        xs = sorted(xs)
        return {"mean_us": round(1000 * sum(xs) / len(xs), 2), "median_us": round(1000 * xs[len(xs) // 2], 2),
                "p10_us": round(1000 * xs[len(xs) // 10], 2), "p90_us": round(1000 * xs[(9 * len(xs)) // 10], 2)}

    stages = {name: stats(stage_ms[i]) for i, name in enumerate(Step.STAGES)}
    median_sum_us = sum(v["median_us"] for v in stages.values())
    lm_mean_s = sum(lm_ms) / len(lm_ms) / 1000.0
    achieved = lm_bytes(w, step.T) / lm_mean_s / 1e9

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": SETTLE_MS,
                   "note": "untimed steps before the warm-up until the GPU has run this long"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "vicuna-7b verify step, batch 1", "B": w["B"], "H": w["H"], "V": w["V"],
                   "K": w["K"], "topk": w["topk"], "T": step.T, "Hq": w["Hq"], "d": w["d"], "L": w["L"],
                   "n_layers": w["n_layers"], "temperature": w["temperature"]},
        "roofline": {"kernel": "lm_head_topk_tree", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "traffic_unit": "bytes per call",
                     "bytes_per_launch": lm_bytes(w, step.T),
                     "mean_launch_us": round(lm_mean_s * 1e6, 2),
                     "launches_timed": len(lm_ms),
                     "timing": "HIP events around the call in one timed step of every %d" % LM_SAMPLE},
        "stages": stages,
        "steps_per_s_stage_medians": round(1e6 / median_sum_us, 2),
        "stages_note": "per-stage statistics from a separate untimed pass of %d steps "
                       "(steps_per_s_stage_medians = 1e6 / the sum of the stage medians, by HIP events); the tree itself "
                       "(medusa_build_tree) is built once per tree spec, per step only its candidates "
                       "and positions are gathered, by the lm_head kernel's last merging workgroup "
                       "(medusa_lm_head_topk_tree)" % nb,
        "tree_candidates_alone_us": round(_time_calls(lambda i: step.run_tree(), 50), 2),
        "build_tree_us": round(_time_calls(lambda i: step.run_build_tree(), 50), 2),
        "tokens_per_step": round(1.0 + sum(a * c for a, c in enumerate(hist)) / sum(hist), 4),
        "accept_len_histogram": hist,
        "accept_len_note": "accepted lengths of the %d rotated logits sets, each with a planted path of "
                           "Binomial(depth, 1/2) steps (the pages' 2.5-3 tokens per step); tokens per step = "
                           "accepted length + 1 (the bonus token)" % Step.NLOGITS,
    }
    if not args.no_graph:
        result["graph"] = graph_timing(step, args.steps)
    if not args.no_base_head:
        result["base_lm_head"] = base_head_timing(step, args.seed, args.steps)
    if not args.no_extra:
        result["nucleus"] = nucleus_timing(step, args.seed, args.steps)
        result["sample_typical"] = sample_typical_timing(step, args.seed, args.steps)
        result["attention_prefix_sweep"] = attention_prefix_sweep(step, args.steps)
        result["vicuna13b"] = vicuna13b(step, args.seed, args.steps)
        result["batch8_33b"] = batch8_33b(step, args.seed, args.steps)
    # a measured streaming-copy rate beside the 8 TB/s peak, taken after
    # every GPU leg (its 2 GiB of buffers are freed before the CPU baseline)
    copy_gbs = copy_peak_gbs()
    result["roofline"].update({
        "copy_peak_gbs": round(copy_gbs, 1), "frac_of_copy_peak": round(achieved / copy_gbs, 4),
        "copy_peak_note": "measured: a 1 GiB device-to-device copy, its read and write bytes by HIP events "
                          "over 20 calls; a copy mixes reads and writes, so a read-only stream such as the "
                          "lm_head's can exceed it"})
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.seed)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
