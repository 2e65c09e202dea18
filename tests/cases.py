"""Parity cases: seeded inputs, oracle expectations, comparisons.

The inputs come from ``synth``; the expected values from ``oracle`` only.
Where a float decides an integer (top-k order, an acceptance test), the
cases redraw inputs until the oracle's decision margins exceed float error,
recording the retry counts.
"""

import numpy as np
import torch

import oracle
import synth


# ------------------------------------------------------------------ compare
def rel_err(got, ref):
    """max |g - o| / max(|o|, rms(o)) over all elements (rms floor for
    near-zero references)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    o = np.asarray(ref, dtype=np.float64).ravel()
    if o.size == 0:
        return 0.0
    floor = max(float(np.sqrt(np.mean(o * o))), 1e-30)
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), floor)))


def tol(dtype):
    """Float tolerance: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs."""
    return 1e-4 if dtype == "f32" else 2e-2


def to_dev(a, dtype=None, device="cuda"):
    """NumPy array -> torch device tensor (uint16 arrays are bf16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def to_host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ------------------------------------------------------------------ heads
def heads_case(w, seed=0, margin=1e-3, max_retries=40):
    """Inputs and oracle results for the heads; each head's lm_head is
    redrawn until the gaps between its top-(k+1) fp64 logits are >= margin
    for every sequence."""
    K, k = w["K"], w["topk"]
    retries = [0] * K
    x = synth.heads_inputs(w, seed=seed, retries=retries)
    for _ in range(max_retries):
        r = oracle.resblock(x["hidden"], x["w1"], x["b1"])
        bad = []
        ref_ids = np.empty((w["B"], K, k), dtype=np.int32)
        ref_vals = np.empty((w["B"], K, k))
        for j in range(K):
            z = oracle.lm_head_logits(r, x["w_lm"], head=j)
            ids, vals = oracle.topk_by_value(z, min(k + 1, w["V"]))
            ref_ids[:, j] = ids[:, :k]
            ref_vals[:, j] = vals[:, :k]
            if np.any(np.diff(-vals, axis=1) < margin):
                bad.append(j)
        if not bad:
            return dict(inputs=x, r=r, topk_ids=ref_ids, topk_logits=ref_vals, retries=retries)
        for j in bad:
            retries[j] += 1
        x = synth.heads_inputs(w, seed=seed, retries=retries)
    raise RuntimeError("no margin after %d redraws" % max_retries)


# ------------------------------------------------------------------ tree
def tree_spec(w, seed=0):
    if w["tree"] == "full":
        return synth.full_tree_choices(w["K"], w["topk"])
    return synth.random_tree_choices(w["depth_counts"], w["topk"], seed=seed, workload_id=w["wid"])


def tree_case(w, seed=0, choices=None):
    choices = tree_spec(w, seed) if choices is None else choices
    ch = synth.choices_array(choices, w["K"])
    ids = synth.topk_ids_input(w, seed=seed)
    root = synth.root_token_input(w, seed=seed)
    plen = synth.prefix_lengths(w, seed=seed)
    ref = oracle.build_tree(ch, w["K"], w["topk"], ids, root, plen)
    return dict(choices=ch, topk_ids=ids, root=root, prefix_len=plen, ref=ref)


# ------------------------------------------------------------------ posterior
def posterior_margins_ok(logits, ref_tree, temperature, eps, delta, rel=1e-3):
    """Decisions far from float error: for every node, the argmax beats the
    runner-up by >= rel (relative to 1) and, in typical mode, every child's
    p differs from its parent's threshold by >= rel * threshold."""
    cand = ref_tree["tree_candidates"]
    parent = ref_tree["parent"]
    B, T, V = logits.shape
    for b in range(B):
        st = oracle.node_statistics(logits[b], temperature)
        x = logits[b].astype(np.float64)
        top2 = -np.sort(-x, axis=1)[:, :2]
        if np.any(top2[:, 0] - top2[:, 1] < rel):
            return False
        if temperature > 0:
            thr = np.minimum(np.float32(eps), np.float32(delta) * np.exp(-st["H"]))
            for c in range(1, T):
                n = parent[c]
                p = np.exp(st["z"][n, cand[b, c]] - st["m"][n]) / st["S"][n]
                if abs(p - thr[n]) < rel * thr[n]:
                    return False
    return True


def non_planted_children_clear(logits, ref_tree, plan):
    """No row outside the planted path has one of its children as argmax."""
    cand, parent = ref_tree["tree_candidates"], ref_tree["parent"]
    B, T, _ = logits.shape
    for b in range(B):
        planted = set()
        if plan[b] is not None:
            p, A = plan[b]
            planted = {int(ref_tree["retrieve"][p, j]) for j in range(A)}
        am = np.argmax(logits[b], axis=1)
        for c in range(1, T):
            n = int(parent[c])
            if n not in planted and cand[b, c] == am[n]:
                return False
    return True


def posterior_case(w, tcase, temperature, seed=0, max_retries=50):
    ref = tcase["ref"]
    for retry in range(max_retries):
        logits, plan = synth.posterior_logits(w, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                              ref["depth"], seed=seed + 1000 * retry)
        if not non_planted_children_clear(logits, ref, plan):
            continue
        if not posterior_margins_ok(logits, ref, temperature, w["eps"], w["delta"]):
            continue
        exp = oracle.evaluate_posterior(logits, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                        temperature, w["eps"], w["delta"])
        return dict(logits=logits, plan=plan, ref=exp, retry=retry)
    raise RuntimeError("no margin after %d redraws" % max_retries)


# ------------------------------------------------------------------ nucleus
def nucleus_margins(logits_row, temperature, top_p, u):
    """How far one node's nucleus decisions sit from a float tie: the
    probability gaps between top_p and the masses just before and at the
    nucleus boundary, and between u * Z and the running masses around the
    drawn token (as fractions of Z).  Returns the smallest."""
    t, q = float(np.float32(temperature)), float(np.float32(top_p))
    z = np.asarray(logits_row, dtype=np.float64) / t
    p = np.exp(z - z.max())
    p /= p.sum()
    V = p.shape[0]
    order = np.lexsort((np.arange(V), -p))
    mass = np.cumsum(p[order])
    k = min(int(np.searchsorted(mass, q, side="left")), V - 1)
    gaps = [mass[k] - q] if k < V - 1 else [1.0]
    if k > 0:
        gaps.append(q - mass[k - 1])
    ids = np.sort(order[:k + 1])
    w = p[ids] / p[ids].sum()
    run = np.cumsum(w)
    target = min(max(float(np.float32(u)), 0.0), 1.0)
    i = int(np.searchsorted(run, target, side="right"))
    if i < len(ids):
        gaps.append(run[i] - target)
        gaps.append(target - (run[i - 1] if i > 0 else 0.0))
    return min(gaps)


def nucleus_case(w, tcase, temperature, top_p, seed=0, tol=1e-5, max_retries=60, plant=None):
    """Planted logits (as for the posterior) and uniforms, redrawn until
    every node's nucleus decisions clear `tol`; with the oracle's verdict."""
    ref = tcase["ref"]
    T = int(np.asarray(ref["tree_candidates"]).shape[1])
    for retry in range(max_retries):
        logits, plan = synth.posterior_logits(w, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                              ref["depth"], seed=seed + 1000 * retry, plant=plant)
        u = synth.node_uniforms(w, T, seed=seed + 1000 * retry)
        ok = all(nucleus_margins(logits[b, n], temperature, top_p, u[b, n]) >= tol
                 for b in range(logits.shape[0]) for n in range(T))
        if not ok:
            continue
        exp = oracle.evaluate_posterior_nucleus(logits, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                                temperature, top_p, u)
        return dict(logits=logits, uniforms=u, plan=plan, ref=exp, retry=retry)
    raise RuntimeError("no margin after %d redraws" % max_retries)


# ------------------------------------------------------------------ decoder
def fitted_heads(model, prompt, n, K, scale=8.0, decoy=0.3, seed=0):
    """Medusa heads fitted in closed form to the oracle's own greedy
    continuation of `prompt`: ResBlocks zero (r = h), and head j's lm_head
    the minimum-norm linear map taking the final hidden state at each
    position t (t = P-1 .. P+n-2) to `scale` on the token at t + j + 2; at a
    `decoy` fraction of positions another token gets 1.3 x scale, so the
    right token is that head's second choice.  Returns bf16 bit arrays
    (w1, b1, w_lm) and the oracle's continuation."""
    cfg = model["cfg"]
    H, V = cfg["H"], cfg["V"]
    cont, _ = oracle.decoder.greedy_decode(model, prompt, n + K + 1)
    seq = list(prompt) + cont
    _, hid = oracle.decoder.forward(model, seq)
    P = len(prompt)
    rows = list(range(P - 1, P - 1 + n))
    Hm = hid[rows]
    G = Hm @ Hm.T + 1e-6 * np.eye(len(rows))
    rng = np.random.default_rng(seed)
    w_lm = np.zeros((K, V, H))
    for j in range(K):
        Y = np.zeros((len(rows), V))
        for r, t in enumerate(rows):
            Y[r, seq[t + j + 2]] = scale
            if rng.random() < decoy:
                other = int(rng.integers(V - 1))
                other += other >= seq[t + j + 2]
                Y[r, other] = 1.3 * scale
        w_lm[j] = np.linalg.solve(G, Y).T @ Hm
    heads = dict(w1=np.zeros((K, H, H), dtype=np.uint16), b1=np.zeros((K, H), dtype=np.uint16),
                 w_lm=synth.bf16_bits(w_lm.astype(np.float32)).reshape(K, V, H))
    return heads, cont[:n]


# ------------------------------------------------------------------ typical acceptance near its threshold
def _chunk_stats(z, chunk):
    """Per-chunk (max, sum exp(z - max), sum (z - max) exp(z - max)) of one
    row, each against its own chunk maximum (the kernel's partial sums)."""
    out = []
    for lo in range(0, z.shape[0], chunk):
        c = z[lo:lo + chunk]
        m = c.max()
        e = np.exp(c - m)
        out.append((m, e.sum(), ((c - m) * e).sum()))
    return out


def merged_entropy(z, chunk, drop_shift=False, batch=None, drop_batch_shift=False):
    """Entropy of softmax(z) assembled from per-chunk partial sums by
    log-sum-exp merging, `batch` chunks at a time, optionally with a planted
    mistake: drop_shift leaves out the (m_c - M) * S_c term of each chunk's
    shifted A, drop_batch_shift the same term of the running sums' rescale
    between batches.  Used only to show that a case can tell a correct
    merge from a broken one."""
    st = _chunk_stats(z, chunk)
    batch = batch or len(st)
    m_run, S_run, A_run = -np.inf, 0.0, 0.0
    for b0 in range(0, len(st), batch):
        part = st[b0:b0 + batch]
        mb = max([m_run] + [p[0] for p in part])
        if m_run != -np.inf:
            w0 = np.exp(m_run - mb)
            A_run = w0 * (A_run + (0.0 if drop_batch_shift else (m_run - mb) * S_run))
            S_run *= w0
        for m, S, A in part:
            w = np.exp(m - mb)
            S_run += w * S
            A_run += w * (A + (0.0 if drop_shift else (m - mb) * S))
        m_run = mb
    return np.log(S_run) - A_run / S_run


def _walk(flags_fn, ret, P, D):
    """Longest leading run of accepted steps per path; lowest-index best."""
    best, best_len = 0, -1
    for p in range(P):
        ell = 0
        for j in range(1, D):
            c = int(ret[p, j])
            if c < 0 or not flags_fn(int(ret[p, j - 1]), c):
                break
            ell += 1
        if ell > best_len:
            best, best_len = p, ell
    return best, best_len


def typical_threshold_case(w, tcase, temperature=0.7, seed=0, chunk=4096, lo=1.05, hi=3.0, max_retries=30,
                           require=("shift",)):
    """Logits [B][T][V] whose typical-acceptance decisions sit close to the
    threshold: every parent's distribution has its entropy branch binding
    (delta * exp(-H) < eps), each child's probability is a factor drawn
    log-uniformly in [lo, hi] above or below its parent's threshold, some
    accepted children have p < eps, and some parent accepts two siblings.
    Rows are N(0, 2.1^2) plus a random offset per `chunk`-wide block of the
    vocabulary, so the mass spreads over blocks whose maxima differ and the
    entropy depends on every block's shifted partial sums; past 8 blocks,
    half the rows lift the later blocks so that their maximum comes after
    the first 8.  Returns the
    logits, the oracle's verdict and, for each of two planted merge
    mistakes, how many child decisions flip and whether the step's output
    changes; the draw is repeated until the output changes under each
    mistake named in `require`."""
    ref = tcase["ref"]
    cand, parent = ref["tree_candidates"], ref["parent"]
    ret, P = ref["retrieve"], int(ref["num_paths"])
    D = ret.shape[1]
    B, T, V = w["B"], int(cand.shape[1]), w["V"]
    t, eps, delta = float(np.float32(temperature)), float(np.float32(w["eps"])), float(np.float32(w["delta"]))
    kids = [[c for c in range(1, T) if int(parent[c]) == n] for n in range(T)]
    for retry in range(max_retries):
        logits = np.empty((B, T, V), dtype=np.float32)
        factors = {}
        for b in range(B):
            g = synth.rng.stream(seed + 1000 * retry, w["wid"], "logits", b, 7)
            off = g.uniform(-1.5, 1.5, size=(V + chunk - 1) // chunk)
            for n in range(T):
                o = off.copy()
                if o.shape[0] > 8 and g.random() < 0.5:
                    o[8:] += 0.7   # the maximum often in a later batch of 8 chunks: the running sums rescale
                x = g.standard_normal(V) * 2.1 + np.repeat(o, chunk)[:V]
                z = x / t
                f = []
                for c in kids[n]:
                    up = g.random() < 0.5
                    r = np.exp(g.uniform(np.log(lo), np.log(hi)))
                    f.append(r if up else 1.0 / r)
                for _ in range(60):
                    m = z.max()
                    e = np.exp(z - m)
                    S = e.sum()
                    H = np.log(S) - ((z - m) * e).sum() / S
                    thr = min(eps, delta * np.exp(-H))
                    for c, fc in zip(kids[n], f):
                        z[int(cand[b, c])] = m + np.log(fc * thr * S)
                logits[b, n] = (z * t).astype(np.float32)
                for c, fc in zip(kids[n], f):
                    factors[(b, c)] = fc
        # verify on the float32 logits with the oracle's statistics
        ok = True
        two = False
        small = False
        flips = {"shift": 0, "batch": 0}
        changed = {"shift": False, "batch": False}
        exp = oracle.evaluate_posterior(logits, cand, ret, P, temperature, w["eps"], w["delta"])
        for b in range(B):
            st = exp["stats"][b]
            x = logits[b].astype(np.float64)
            top2 = -np.sort(-x, axis=1)[:, :2]
            if np.any(top2[:, 0] - top2[:, 1] < 1e-3):
                ok = False
            for n in range(T):
                if not kids[n]:
                    continue
                if delta * np.exp(-st["H"][n]) >= eps:
                    ok = False
                acc = 0
                for c in kids[n]:
                    p = np.exp(st["z"][n, cand[b, c]] - st["m"][n]) / st["S"][n]
                    ratio = p / st["thr"][n]
                    if not (lo / 1.01 <= ratio <= hi * 1.01 or 1 / (hi * 1.01) <= ratio <= 1.01 / lo):
                        ok = False
                    if ratio > 1:
                        acc += 1
                        small = small or p < eps
                two = two or acc >= 2
            for name, kw in (("shift", dict(drop_shift=True, batch=8)), ("batch", dict(drop_batch_shift=True, batch=8))):
                thr_w = np.array([min(eps, delta * np.exp(-merged_entropy(st["z"][n], chunk, **kw)))
                                  for n in range(T)])

                def flag(n, c, thr_n=None):
                    p = np.exp(st["z"][n, cand[b, c]] - st["m"][n]) / st["S"][n]
                    return np.float32(p) > np.float32(thr_n[n] if thr_n is not None else st["thr"][n])

                flips[name] += sum(flag(n, c) != flag(n, c, thr_w) for n in range(T) for c in kids[n])
                bw, lw = _walk(lambda n, c: flag(n, c, thr_w), ret, P, D)
                if (bw, lw) != (int(exp["best_path"][b]), int(exp["accept_len"][b])):
                    changed[name] = True
        if ok and two and small and all(changed[r] for r in require):
            return dict(logits=logits, ref=exp, retry=retry, flips=flips, changed=changed, factors=factors)
    raise RuntimeError("no near-threshold case after %d redraws" % max_retries)


# ------------------------------------------------------------------ sampled next token
def typical_sample_robust(row, temperature, eps, delta, u, rel=1e-5, thr_rel=1e-3):
    """Whether one typical-mode draw is decided far from float error: the
    draw is the same with every near-threshold token (|p - thr| < thr_rel *
    thr) counted in and counted out, and u times the allowed mass lies at
    least rel of that mass away from every running-sum boundary."""
    from oracle import sampling as smp
    t = float(np.float32(temperature))
    z = np.asarray(row, dtype=np.float64) / t
    e = np.exp(z - z.max())
    S = e.sum()
    H = np.log(S) - ((z - z.max()) * e).sum() / S
    thr = min(float(np.float32(eps)), float(np.float32(delta)) * np.exp(-H))
    p = e / S
    near = np.abs(p - thr) < thr_rel * thr
    draws = []
    for keep in (p > thr) | near, (p > thr) & ~near:
        ids = np.flatnonzero(keep)
        w = p[ids]
        target = float(np.float32(u)) * w.sum()
        run = np.cumsum(w)
        if np.min(np.abs(run - target)) < rel * w.sum():
            return False
        i = int(np.searchsorted(run, target, side="right"))
        draws.append(int(ids[min(i, len(ids) - 1)]))
    return draws[0] == draws[1] == smp.typical_sample(row, temperature, eps, delta, u)
