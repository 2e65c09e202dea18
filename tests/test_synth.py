"""The synthetic-input recipes: determinism, shapes and encodings."""

import numpy as np

import synth


def test_streams_are_deterministic_and_distinct():
    a = synth.normal_f32(0, 1, "w1", (0,), 3 << 20)
    b = synth.normal_f32(0, 1, "w1", (0,), 3 << 20)
    c = synth.normal_f32(0, 1, "w1", (1,), 3 << 20)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert abs(float(a.std()) - 1.0) < 0.01


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, np.inf], dtype=np.float32)
    bits = synth.bf16_bits(x)
    back = synth.bf16_to_f32(bits)
    # 1 + 2^-8 is the tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-9 rounds up
    assert back.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -7, -2.5]
    assert np.isinf(back[5])
    nanbits = synth.bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(synth.bf16_to_f32(nanbits)[0])


def test_random_tree_shape():
    w = synth.workload("vicuna-7b")
    ch = synth.random_tree_choices(w["depth_counts"], w["topk"], seed=3, workload_id=w["wid"])
    assert len(ch) == 63
    depths = np.bincount([len(t) for t in ch])
    assert depths.tolist() == [0, 10, 20, 16, 10, 7]
    assert all(0 <= r < 10 for t in ch for r in t)
    assert len(set(ch)) == 63


def test_heads_inputs_rms_normalised_bf16():
    w = synth.workload("vicuna-7b", H=256, V=300, K=2)
    x = synth.heads_inputs(w, seed=0)
    assert x["hidden"].dtype == np.uint16 and x["w_lm"].shape == (2, 300, 256)
    h = synth.bf16_to_f32(x["hidden"]).astype(np.float64)
    assert abs(float(np.sqrt(np.mean(h * h))) - 1.0) < 0.01
    y = synth.heads_inputs(w, seed=0, retries=[0, 1])
    assert np.array_equal(x["w_lm"][0], y["w_lm"][0])
    assert not np.array_equal(x["w_lm"][1], y["w_lm"][1])


def test_attention_inputs_poison_and_rope_norm():
    w = synth.workload("tiny-f32", S_max=160)
    depth = np.array([0, 1, 1, 2])
    x = synth.attention_inputs(w, depth, np.array([128]), seed=0)
    kc = x["k_cache"]
    assert np.all(np.isnan(kc[0, :, 132:]))
    assert not np.any(np.isnan(kc[0, :, :132]))
    # rotation preserves norms
    rows = np.random.default_rng(0).standard_normal((5, 64))
    rot = synth.rope_rotate(rows, np.arange(5) * 37)
    assert np.allclose(np.linalg.norm(rot, axis=1), np.linalg.norm(rows, axis=1))
