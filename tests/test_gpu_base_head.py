"""GPU parity of the base lm_head over the tree nodes against the oracle.

logits = hidden . W^T with bf16 inputs: every product is exact in float32,
so the kernel's float32 sums stay within 1e-4 max relative error of the
fp64 oracle (tighter than the 2e-2 bf16 bar).  Both weight layouts: row-
major and packed (the packed bytes themselves are checked bit for bit
against the layout the header documents, restated here with NumPy).
Sizes: ragged M (partial M tiles), ragged V (partial vocab blocks and
tiles), H below and past the 256-element K chunk with a tail and a partial
32-element k step, the smallest shape, and the Vicuna-7B tree (64 nodes,
H 4096, V 32000).

The fused form (medusa_base_posterior: per-row statistics and the
children's logits in the GEMM epilogue, the logits never written) returns
best path, accepted length and next token equal to the oracle's acceptance
test on the same planted inputs: greedy and typical, both weight layouts,
one sequence and several whose 64-row tiles straddle sequence boundaries.
Greedy decisions follow from the raw logits alone, which the fused and the
unfused forms compute with the same MFMA accumulation, so on unplanted
inputs the two agree exactly as well.
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(M, H, V, seed):
    x = synth.base_head_inputs(M, H, V, seed=seed)
    return x["hidden"], x["w_base"]


def _packed_reference(w):
    """The documented packed layout of bf16 bits w [V][H]: for tile t, k step
    s and lane l = 16 g + n, 8 elements W[16 t + n][32 s + 8 g ..] (zero past
    V or H, tile count padded to even), ordered step, tile pair, tile within
    the pair, lane."""
    V, H = w.shape
    Vt, S = (V + 31) // 32 * 2, (H + 31) // 32
    pad = np.zeros((Vt * 16, S * 32), dtype=np.uint16)
    pad[:V, :H] = w
    t = pad.reshape(Vt // 2, 2, 16, S, 4, 8)          # [pair][q][n][s][g][e]
    return np.ascontiguousarray(t.transpose(3, 0, 1, 4, 2, 5)).reshape(-1)   # [s][pair][q][g][n][e]


@pytest.mark.parametrize("V,H", [(1, 8), (17, 40), (300, 72), (1000, 264)])
def test_base_lm_head_pack_layout(gpu_device, V, H):
    _, w = _inputs(1, H, V, seed=V * H)
    got = md.medusa_base_lm_head_pack(to_dev(w))
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _packed_reference(w))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M,H,V", [
    (1, 8, 1),          # smallest shape
    (5, 72, 300),       # one partial K chunk, partial vocab block, partial M tile
    (64, 520, 1000),    # K tail past two chunks, ragged V
    (130, 264, 777),    # three M tiles
    (16, 4096, 2051),   # full-width rows, ragged V
    (7, 40, 33),        # partial 32-element k step, partial 16-row tile
])
def test_base_lm_head_matches_oracle(gpu_device, M, H, V, packed):
    h, w = _inputs(M, H, V, seed=M + H + V)
    print("case", M, H, V, packed, flush=True)
    wd = to_dev(w)
    if packed:
        wd = md.medusa_base_lm_head_pack(wd)
    got = md.medusa_base_lm_head(to_dev(h), wd, V=V)
    torch.cuda.synchronize()
    ref = oracle.base_logits(h, w)
    assert rel_err(to_host(got), ref) < 1e-4


@pytest.mark.parametrize("packed", [False, True])
def test_base_lm_head_vicuna7b_tree(gpu_device, packed):
    # the 64 tree nodes of one sequence against the 32000 x 4096 lm_head,
    # through the [B][T][H] form of the binding
    M, H, V = 64, 4096, 32000
    h, w = _inputs(M, H, V, seed=0)
    wd = to_dev(w)
    if packed:
        wd = md.medusa_base_lm_head_pack(wd)
    got = md.medusa_base_lm_head(to_dev(h).view(1, M, H), wd, V=V)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (1, M, V)
    ref = oracle.base_logits(h, w)
    assert rel_err(to_host(got).reshape(M, V), ref) < 1e-4


def test_base_lm_head_writes_only_its_rows(gpu_device):
    # an output larger than M x V keeps its tail: rows past M are never written
    M, H, V = 3, 64, 200
    h, w = _inputs(M, H, V, seed=9)
    big = torch.full((M + 2, V), 7.0, dtype=torch.float32, device=gpu_device)
    hd, wd = to_dev(h), to_dev(w)   # held until the kernel has run
    rc = md.lib.medusa_base_lm_head(md.MEDUSA_BF16, M, H, V, hd.data_ptr(), wd.data_ptr(), 0, big.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    assert rel_err(out[:M], oracle.base_logits(h, w)) < 1e-4
    assert np.all(out[M:] == 7.0)


_CASES = {}


def _base_posterior_case(w, temperature, seed=0, max_retries=20, scale=20.0, h_std=1.0):
    """Tree, planted hidden states and the oracle's verdict; redrawn until
    the decisions clear float error (as for the posterior on given logits).
    Cached per (shape, temperature, seed, generator settings)."""
    key = (w["B"], w["H"], w["V"], w["K"], w["topk"], w["tree"], temperature, seed, scale, h_std)
    if key in _CASES:
        return _CASES[key]
    from cases import non_planted_children_clear, posterior_margins_ok, tree_case
    tcase = tree_case(w, seed=seed)
    ref = tcase["ref"]
    for retry in range(max_retries):
        x = synth.base_posterior_inputs(w, ref["tree_candidates"], ref["retrieve"], ref["num_paths"],
                                        seed=seed + 1000 * retry, scale=scale, h_std=h_std)
        B, T, H = x["hidden"].shape
        z = oracle.base_logits(x["hidden"].reshape(B * T, H), x["w_base"]).reshape(B, T, -1).astype(np.float32)
        if not non_planted_children_clear(z, ref, x["plan"]):
            continue
        if not posterior_margins_ok(z, ref, temperature, w["eps"], w["delta"]):
            continue
        exp = oracle.base_posterior(x["hidden"], x["w_base"], ref["tree_candidates"], ref["retrieve"],
                                    ref["num_paths"], temperature, w["eps"], w["delta"])
        _CASES[key] = (tcase, x, exp, retry)
        return _CASES[key]
    raise RuntimeError("no margin after %d redraws" % max_retries)


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_base_lm_head_then_posterior_matches_oracle(gpu_device, temperature):
    # the base logits of the 64-node tree (H 1024, V 8000, packed weights;
    # the full 4096 x 32000 GEMM has its own parity test) feed the acceptance
    # test; best path, accepted length and next token equal the oracle's on
    # the same planted inputs
    w = synth.workload("vicuna-7b", H=1024, V=8000)
    tcase, x, exp, retry = _base_posterior_case(w, temperature)
    print("retry", retry, "plan", x["plan"], "expected", exp["accept_len"], flush=True)
    ref = tcase["ref"]
    B, T, H = x["hidden"].shape
    V = x["w_base"].shape[0]
    wp = md.medusa_base_lm_head_pack(to_dev(x["w_base"]))
    logits = md.medusa_base_lm_head(to_dev(x["hidden"]), wp, V=V)
    got = md.medusa_evaluate_posterior(logits, to_dev(ref["tree_candidates"]), to_dev(ref["retrieve"]),
                                       to_dev(np.array([ref["num_paths"]], dtype=np.int32)), temperature,
                                       w["eps"], w["delta"])
    torch.cuda.synchronize()
    for key in ("best_path", "accept_len", "next_token"):
        assert np.array_equal(got[key].cpu().numpy(), exp[key]), key
    assert int(exp["accept_len"][0]) == x["plan"][0][1]


def _fused(x, ref, w, temperature, packed):
    V = x["w_base"].shape[0]
    wd = to_dev(x["w_base"])
    if packed:
        wd = md.medusa_base_lm_head_pack(wd)
    args = (to_dev(x["hidden"]), wd, to_dev(ref["tree_candidates"]), to_dev(ref["retrieve"]),
            to_dev(np.array([ref["num_paths"]], dtype=np.int32)))
    got = md.medusa_base_posterior(*args, temperature, w["eps"], w["delta"], V=V)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in got.items()}


# (workload overrides, generator settings)
_FUSED_SHAPES = {
    # the 64-node Vicuna-7B tree, one sequence, at the full 4096 x 32000
    # lm_head (the shape the fused form is timed at); node logits of std
    # about 1.3, so at temperature 0.7 the entropy branch sets the
    # thresholds and decides the unplanted children
    "vicuna7b-full": (dict(), dict()),
    # the same tree with H and V cut
    "vicuna7b-tree": (dict(H=1024, V=8000), dict()),
    # 5 sequences of 15 nodes: M = 75, the first 64-row tile holds five
    # sequences, the second a partial one; ragged V (last block 57 wide)
    "b5-full15": (dict(B=5, K=3, topk=2, tree="full", H=512, V=3001), dict()),
    # 3 sequences of the 64-node tree: tiles aligned with sequences; H with a
    # partial K chunk
    "b3-tree": (dict(B=3, H=520, V=4100), dict()),
    # peaked nodes (logit std about 3): low entropy, so typical acceptance
    # thresholds sit among the children's probabilities and decide
    "b4-tree-peaked": (dict(B=4, H=512, V=3001), dict(h_std=6.0, scale=80.0)),
}


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("temperature", [0.0, 0.7])
@pytest.mark.parametrize("shape", sorted(_FUSED_SHAPES))
def test_base_posterior_fused_matches_oracle(gpu_device, shape, temperature, packed):
    over, gen = _FUSED_SHAPES[shape]
    w = synth.workload("vicuna-7b", **over)
    tcase, x, exp, retry = _base_posterior_case(w, temperature, **gen)
    print("case", shape, temperature, packed, "retry", retry, "plan", x["plan"], "expected", exp["accept_len"],
          flush=True)
    got = _fused(x, tcase["ref"], w, temperature, packed)
    for key in ("best_path", "accept_len", "next_token"):
        assert np.array_equal(got[key], exp[key]), key
    if temperature == 0.0:
        assert [int(a) for a in exp["accept_len"]] == [p[1] for p in x["plan"]]


@pytest.mark.parametrize("shape", sorted(_FUSED_SHAPES))
def test_base_posterior_fused_equals_unfused_greedy(gpu_device, shape):
    # unplanted hidden states: arbitrary argmaxes, decided on logits both
    # forms compute identically
    over, gen = _FUSED_SHAPES[shape]
    w = synth.workload("vicuna-7b", **over)
    ref = tree_case_ref(w)
    x = synth.base_posterior_inputs(w, ref["tree_candidates"], ref["retrieve"], ref["num_paths"], seed=77,
                                    plant=False, h_std=gen.get("h_std", 1.0))
    V = x["w_base"].shape[0]
    got = _fused(x, ref, w, 0.0, True)
    wp = md.medusa_base_lm_head_pack(to_dev(x["w_base"]))
    logits = md.medusa_base_lm_head(to_dev(x["hidden"]), wp, V=V)
    un = md.medusa_evaluate_posterior(logits, to_dev(ref["tree_candidates"]), to_dev(ref["retrieve"]),
                                      to_dev(np.array([ref["num_paths"]], dtype=np.int32)), 0.0, w["eps"],
                                      w["delta"])
    torch.cuda.synchronize()
    for key in ("best_path", "accept_len", "next_token"):
        assert np.array_equal(got[key], un[key].cpu().numpy()), key


def tree_case_ref(w, seed=0):
    from cases import tree_case
    return tree_case(w, seed=seed)["ref"]


@pytest.mark.parametrize("M,H,V", [
    (1, 2816, 1024),    # eleven chunks in eleven slices (the tiny model's down projection)
    (15, 1024, 3072),   # four slices, a 15-node tree through QKV
    (32, 1032, 300),    # a partial last chunk in the last slice, ragged V
    (64, 4096, 5632),   # the widest M that splits
    (65, 1024, 1024),   # two M tiles: no split
    (1, 1024, 32000),   # 250 vocabulary blocks: no split
    (3, 200, 64),       # one chunk: nothing to split
])
def test_linear_matches_oracle_and_is_deterministic(gpu_device, M, H, V):
    h, w = _inputs(M, H, V, seed=3 * M + H + V)
    print("case", M, H, V, md.medusa_linear_workspace(M, H, V), flush=True)
    wp = md.medusa_base_lm_head_pack(to_dev(w))
    x = to_dev(h)
    a = md.medusa_linear(x, wp, V)
    b = md.medusa_linear(x, wp, V)
    torch.cuda.synchronize()
    assert rel_err(to_host(a), oracle.base_logits(h, w)) < 1e-4
    assert torch.equal(a, b)
