"""GPU parity of medusa_tree_attention against the oracle.

Slots past each sequence's tree hold NaN, so a read beyond L + T shows up as
NaN in the output.  Cases: the tiny fp32 workload, bf16 shapes that are
ragged against the 64-key chunk and 256-key split (including L = 0 and a
prefix shorter than one split), trees larger than one 64-query block, the
full Vicuna-7B layer at every swept prefix, a batch whose sequences get
different split counts, and the Vicuna-33B batch of 8 (one long split per
sequence and head).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_medusa_amd as md
import synth
from cases import rel_err, tol, to_dev, to_host, tree_case

pytestmark = pytest.mark.gpu


def _run_case(w, seed=0, choices=None, plen=None):
    tc = tree_case(w, seed=seed, choices=choices)
    ref_tree = tc["ref"]
    plen = tc["prefix_len"] if plen is None else np.asarray(plen, dtype=np.int32)
    x = synth.attention_inputs(w, ref_tree["depth"], plen, seed=seed)
    scale = 1.0 / math.sqrt(w["d"])
    ref = oracle.tree_attention(x["q"], x["k_cache"], x["v_cache"], plen, ref_tree["tree_mask"], scale)
    out = md.medusa_tree_attention(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(plen),
                                   to_dev(ref_tree["tree_mask"]), scale)
    torch.cuda.synchronize()
    got = to_host(out)
    if got.dtype == np.uint16:
        got = synth.bf16_to_f32(got)
    assert not np.any(np.isnan(got))
    err = rel_err(got, ref)
    print("attention max rel err %.3e" % err, flush=True)
    assert err < tol(w["dtype"])
    return err


def test_attention_tiny_f32(gpu_device):
    _run_case(synth.workload("tiny-f32"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [0, 1, 100, 255, 256, 300, 700])
def test_attention_bf16_ragged(gpu_device, d, L):
    w = synth.workload("tiny-f32", dtype="bf16", d=d, Hq=3, S_max=L + 15 + 5)
    _run_case(w, seed=L, plen=[L])


def test_attention_f32_d128_batch(gpu_device):
    w = synth.workload("tiny-f32", d=128, B=3, S_max=600, L_range=(0, 580))
    _run_case(w, seed=4)


@pytest.mark.parametrize("counts", [(10, 20, 30, 20, 19), (40, 60, 60, 40, 25, 15, 10, 5)])
def test_attention_large_trees(gpu_device, counts):
    # 100 and 256 nodes: two and four 64-query blocks
    K = len(counts)
    w = synth.workload("vicuna-7b", K=K, topk=64, depth_counts=counts, Hq=4, L=520, S_max=520 + 300)
    _run_case(w, seed=len(counts))


@pytest.mark.parametrize("L", [512, 1024, 2048, 4096])
def test_attention_vicuna7b(gpu_device, L):
    w = synth.workload("vicuna-7b", L=L, S_max=L + 64)
    _run_case(w, seed=0)


def test_attention_batch_mixed_split_counts(gpu_device):
    # four sequences at the 7B layer shape with max_slots 2120: the launch
    # takes splits of 1060 keys, so the longest sequence (2120 keys) gets two
    # splits, merged by the second kernel, and the others one, written
    # directly by the first
    w = synth.workload("vicuna-7b", B=4, L=2048, S_max=2120)
    _run_case(w, seed=2, plen=[2056, 1500, 1999, 610])


@pytest.mark.slow
def test_attention_vicuna33b_batch8(gpu_device):
    w = synth.workload("vicuna-33b-b8")
    _run_case(w, seed=0)


def test_attention_vicuna13b(gpu_device):
    # 40 heads x 128 at prefix 2048
    w = synth.workload("vicuna-13b")
    _run_case(w, seed=1)
