"""GPU parity of the Medusa heads (ResBlock + lm_head + top-k) against the oracle.

Top-k ids are compared bit for bit (inputs redrawn until the oracle's top-k
gaps exceed 1e-3); r, top-k logits and full logits within 1e-4 (fp32) or
2e-2 (bf16) max relative error.  Sizes: the tiny fp32 workload, ragged bf16
shapes spanning several tiles, workgroups and a partial K step, and the full
Vicuna-7B (batch 1) and Vicuna-33B (batch 8) head shapes.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_medusa_amd as md
import synth
from cases import heads_case, rel_err, tol, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(case, w, keep_logits=True, split=False):
    x = case["inputs"]
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    if split:
        r = md.medusa_resblock(h, w1, b1)
        out = md.medusa_lm_head_topk(r, wlm, w["topk"], keep_logits=keep_logits)
        out["r"] = r
    else:
        out = md.medusa_heads(h, w1, b1, wlm, w["topk"], keep_logits=keep_logits, keep_r=True)
    torch.cuda.synchronize()
    return {k: (to_host(v) if v is not None else None) for k, v in out.items()}


def _check(case, got, w, check_logits=True):
    print("retries", case["retries"], flush=True)
    assert rel_err(got["r"], case["r"]) < tol(w["dtype"])
    assert np.array_equal(got["topk_ids"], case["topk_ids"])
    assert rel_err(got["topk_logits"], case["topk_logits"]) < tol(w["dtype"])
    if check_logits and got.get("logits") is not None:
        import oracle
        z = oracle.lm_head_logits(case["r"], case["inputs"]["w_lm"])
        assert rel_err(got["logits"], z) < tol(w["dtype"])


def test_heads_tiny_f32(gpu_device):
    w = synth.workload("tiny-f32")
    case = heads_case(w, seed=0)
    _check(case, _run(case, w), w)


@pytest.mark.parametrize("B,H,V,K,k", [
    (1, 264, 1000, 3, 5),      # H not a multiple of 32: partial last K step
    (3, 1048, 5003, 2, 7),     # odd V: ragged last tile and workgroup
    (8, 520, 777, 4, 16),      # full MFMA M tile
    (9, 264, 2000, 2, 3),      # two M tiles
    (16, 136, 300, 8, 64),     # maximum batch, heads and top-k
    (1, 8, 64, 1, 64),         # k == V
])
def test_heads_bf16_ragged(gpu_device, B, H, V, K, k):
    # with H <= 1048 the float32 error of a logit is below 1e-7, so a 1e-5
    # gap is a 100x margin; it lets k approach V without endless redraws
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=B * 7 + K, margin=1e-5, max_retries=400)
    _check(case, _run(case, w, split=(B % 2 == 1)), w)


def test_heads_f32_batch(gpu_device):
    w = synth.workload("tiny-f32", B=5, H=132, V=333, K=2, topk=9)
    case = heads_case(w, seed=3)
    _check(case, _run(case, w), w)


def test_heads_vicuna7b(gpu_device):
    w = synth.workload("vicuna-7b")
    case = heads_case(w, seed=0)
    _check(case, _run(case, w, keep_logits=False), w)


def test_heads_repeat_calls_are_stable(gpu_device):
    # the same call three times on one cached workspace gives the same answer
    w = synth.workload("vicuna-7b", B=2, H=256, V=4000, K=3, topk=10)
    case = heads_case(w, seed=11)
    for _ in range(3):
        _check(case, _run(case, w, keep_logits=False), w, check_logits=False)


def test_heads_back_to_back_inputs_share_workspace(gpu_device):
    # different inputs in turn (A, B, A, B) through one cached workspace:
    # the in-kernel merge (taken here: 5 heads of 50 workgroups x 4 lists x
    # 10 = 2000 candidates) must read the lists of the running call, never a
    # previous call's, and leave its arrival counts ready for the next
    w = synth.workload("vicuna-7b", B=1, H=512, V=6000, K=5, topk=10)
    a = heads_case(w, seed=21)
    b = heads_case(w, seed=22)
    assert not np.array_equal(a["topk_ids"], b["topk_ids"])
    for case in (a, b, a, b):
        _check(case, _run(case, w, keep_logits=False, split=True), w, check_logits=False)


@pytest.mark.parametrize("B,H,V,K,k", [
    (1, 6656, 3001, 2, 10),    # 13 row steps of 512 (the 33B hidden size, batch 1)
    (2, 8192, 2000, 1, 8),     # 16 row steps, two sequences per wave
    (1, 8200, 700, 2, 5),      # past 16 row steps: the skinny-GEMM path at batch 1
])
def test_heads_bf16_wide_rows(gpu_device, B, H, V, K, k):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=H + B)
    _check(case, _run(case, w), w)


@pytest.mark.slow
def test_heads_vicuna33b_batch8(gpu_device):
    w = synth.workload("vicuna-33b-b8")
    case = heads_case(w, seed=0)
    _check(case, _run(case, w, keep_logits=False), w)


def _run_packed(case, w, keep_logits=True):
    x = case["inputs"]
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    r = md.medusa_resblock(h, w1, b1)
    packed = md.medusa_heads_pack(wlm)
    out = md.medusa_lm_head_topk_packed(r, packed, w["V"], w["topk"], keep_logits=keep_logits)
    out["r"] = r
    torch.cuda.synchronize()
    return {k: (to_host(v) if v is not None else None) for k, v in out.items()}


@pytest.mark.parametrize("B,H,V,K,k", [
    (1, 264, 1000, 3, 5),      # batch 1, partial last K chunk
    (3, 1048, 5003, 2, 7),     # odd V: ragged last vocabulary block
    (8, 520, 777, 4, 16),
    (16, 136, 300, 5, 64),     # maximum batch and top-k
    (1, 8, 64, 1, 64),         # k == V
])
def test_heads_packed_bf16(gpu_device, B, H, V, K, k):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=B * 5 + K, margin=1e-5, max_retries=400)
    _check(case, _run_packed(case, w), w)


def test_heads_packed_matches_row_major(gpu_device):
    # packed and row-major weights give identical top-k ids and logits on
    # the same r (same products, same summation order per output)
    w = synth.workload("vicuna-7b", B=4, H=1024, V=9000, K=3, topk=10)
    case = heads_case(w, seed=31)
    x = case["inputs"]
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    r = md.medusa_resblock(h, w1, b1)
    a = md.medusa_lm_head_topk(r, wlm, 10, keep_logits=True)
    b = md.medusa_lm_head_topk_packed(r, md.medusa_heads_pack(wlm), 9000, 10, keep_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(a["topk_ids"], b["topk_ids"])
    assert rel_err(to_host(b["topk_logits"]), to_host(a["topk_logits"])) < 1e-6
    assert rel_err(to_host(b["logits"]), to_host(a["logits"])) < 1e-6


@pytest.mark.slow
def test_heads_packed_vicuna33b_batch8(gpu_device):
    w = synth.workload("vicuna-33b-b8")
    case = heads_case(w, seed=0)
    _check(case, _run_packed(case, w, keep_logits=False), w)


def _run_heads_packed(case, w, keep_logits=True):
    x = case["inputs"]
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    out = md.medusa_heads_packed(h, md.medusa_heads_pack(w1), b1, md.medusa_heads_pack(wlm), w["V"], w["topk"],
                                 keep_logits=keep_logits, keep_r=True)
    torch.cuda.synchronize()
    return {k: (to_host(v) if v is not None else None) for k, v in out.items()}


# margins: the logit error of the hi/lo planes grows like sqrt(H) (about
# 4e-6 at H = 2056, 1e-5 at H = 8192), so wide rows take wider gaps
@pytest.mark.parametrize("B,H,V,K,k,margin", [
    (1, 264, 1000, 3, 5, 1e-5),       # two chunks: one full, one partial
    (3, 1048, 5003, 2, 7, 1e-5),      # five chunks in slices, odd V
    (8, 520, 777, 4, 16, 1e-5),
    (16, 2056, 3000, 5, 16, 1e-4),    # maximum batch, nine chunks in five slices
    (2, 8192, 2000, 1, 8, 1e-3),      # 32 chunks: eight slices of four
    (1, 8, 64, 1, 64, 1e-5),          # k == V, H of one MFMA piece
])
def test_heads_packed_both_stages(gpu_device, B, H, V, K, k, margin):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=B * 3 + K, margin=margin, max_retries=400)
    _check(case, _run_heads_packed(case, w), w)


@pytest.mark.slow
def test_heads_packed_both_stages_vicuna33b_batch8(gpu_device):
    w = synth.workload("vicuna-33b-b8")
    case = heads_case(w, seed=1)
    _check(case, _run_heads_packed(case, w, keep_logits=False), w)


def test_heads_vicuna13b(gpu_device):
    # H 5120: ten 512-element row steps, the row-diagonal kernels' ragged case
    w = synth.workload("vicuna-13b")
    case = heads_case(w, seed=0)
    _check(case, _run(case, w, keep_logits=False), w)


@pytest.mark.parametrize("H", [4096, 5120, 6656, 8192])
def test_heads_logit_error_from_r_planes(gpu_device, H):
    # r enters the lm_head GEMV as two bf16 planes (hi = bf16(r), lo =
    # bf16(r - hi)), about 16 significant bits of the float32 r; the logits
    # of that product stay within the float32 bar (1e-4) of the fp64 oracle's
    # z = Wlm r at the Vicuna-7B, 13B and 33B hidden sizes and at 8192, the
    # largest hidden size the row-diagonal kernels take
    import oracle
    w = synth.workload("vicuna-7b", H=H, K=2)
    x = synth.heads_inputs(w, seed=H)
    h, w1, b1, wlm = (to_dev(x[n]) for n in ("hidden", "w1", "b1", "w_lm"))
    got = md.medusa_heads(h, w1, b1, wlm, w["topk"], keep_logits=True, keep_r=True)
    torch.cuda.synchronize()
    r = oracle.resblock(x["hidden"], x["w1"], x["b1"])
    z = np.stack([oracle.lm_head_logits(r, x["w_lm"], head=j) for j in range(w["K"])], axis=1)
    gl = to_host(got["logits"]).astype(np.float64)
    err = rel_err(gl, z)
    abs_err = float(np.max(np.abs(gl - z)))
    print("H %d logits max rel err %.3e, max abs err %.3e (logit std %.3f)" % (H, err, abs_err, float(z.std())),
          flush=True)
    assert err < 1e-4


# The row-diagonal lm_head with its in-kernel merge (bf16, batch <= 2, lists
# x top-k <= 2048) and rows of H > 2048 hands the last seventh of each head's
# rows out in blocks of four from a device-scope counter.  Cases: a pool of a
# few blocks after one static row per wave, a row count below the number of
# waves (every row from the pool, a partial last block), a ragged V at batch
# 2, eight heads at top-16, and H 2560 (the smallest row length that takes
# the pool).
@pytest.mark.parametrize("B,H,V,K,k", [
    (1, 4096, 300, 5, 10),
    (1, 2560, 150, 5, 10),
    (2, 4096, 5003, 5, 10),
    (1, 3072, 4001, 8, 16),
    (1, 2560, 7000, 4, 8),
])
def test_heads_dynamic_row_pool(gpu_device, B, H, V, K, k):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=H + V + K, margin=1e-5, max_retries=400)
    _check(case, _run(case, w, split=(B == 1)), w)


def test_heads_dynamic_row_pool_calls_in_turn(gpu_device):
    # inputs A, B, A, B through one workspace at a pool shape: each call's
    # counters start at zero (the merging workgroups reset them) and every
    # row is taken exactly once
    w = synth.workload("vicuna-7b", B=1, H=4096, V=3000, K=5, topk=10)
    a = heads_case(w, seed=41, margin=1e-5, max_retries=400)
    b = heads_case(w, seed=42, margin=1e-5, max_retries=400)
    assert not np.array_equal(a["topk_ids"], b["topk_ids"])
    for case in (a, b, a, b):
        _check(case, _run(case, w, keep_logits=True), w)


def _pool_shapes(n, seed=2024):
    """Seeded random shapes that take the lm_head's dynamic row pool (bf16,
    batch <= 2, H > 2048, lists x top-k within the in-kernel merge)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B = int(rng.integers(1, 3))
        H = int(rng.integers(2056, 6145)) // 8 * 8
        K = int(rng.integers(3, 9))
        V = int(rng.integers(64, 8001))
        lists = 4 * max(1, min(256 // K, -(-V // 4)))
        kmax = min(2048 // lists, 64, V)
        if kmax < 1:
            continue
        k = int(rng.integers(1, kmax + 1))
        out.append((B, H, V, K, k))
    return out


@pytest.mark.parametrize("B,H,V,K,k", _pool_shapes(12))
def test_heads_dynamic_row_pool_random_shapes(gpu_device, B, H, V, K, k):
    w = synth.workload("vicuna-7b", B=B, H=H, V=V, K=K, topk=k)
    case = heads_case(w, seed=B + H + V + K + k, margin=1e-5, max_retries=400)
    _check(case, _run(case, w, keep_logits=True), w)
