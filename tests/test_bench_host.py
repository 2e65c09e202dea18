"""Host-side pieces of bench.py (no GPU): the roofline's algorithmic bytes,
the traffic figure read from the committed counter summary only while it
matches the heads source, the attention bytes of a layer, and the refusal of
more than one GPU."""

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_lm_bytes_is_weights_inputs_and_outputs():
    w = synth.workload("vicuna-7b")
    # 5 heads x 32000 x 4096 bf16 weights, r in float32, top-10 (id, logit) pairs out;
    # the 64-node tree gather: tree_indices and depth, root and prefix length,
    # one top-k id per node in, candidates and positions out (int32)
    gather = (2 * 64 + 2 * 1 + 3 * 64) * 4
    assert bench.lm_bytes(w, 64) == 5 * 32000 * 4096 * 2 + 5 * 4096 * 4 + 5 * 10 * 8 + gather == 1310803608


def test_measured_traffic_follows_the_heads_source(tmp_path, monkeypatch):
    src = tmp_path / "heads.hip"
    src.write_bytes(b"kernel source")
    prof = tmp_path / "traffic.md"
    sha = hashlib.sha256(b"kernel source").hexdigest()
    prof.write_text("x\ntraffic_bytes_per_call: 1314322809\nheads_hip_sha256: %s\n" % sha)
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    monkeypatch.setattr(bench, "HEADS_SOURCE", str(src))
    assert bench.measured_traffic() == 1314322809
    src.write_bytes(b"kernel source, changed")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout
