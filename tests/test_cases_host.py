"""CPU checks of the parity-case builders themselves: the chunk-merge
entropy used to prove a case's sensitivity equals the oracle's entropy when
nothing is dropped, and the near-threshold typical case has the properties
its GPU test relies on."""

import numpy as np

import oracle
import synth
from cases import merged_entropy, tree_case, typical_threshold_case


def test_merged_entropy_without_mistake_is_the_entropy():
    rng = np.random.default_rng(1)
    for V in (100, 4096, 9000, 40000):
        z = rng.standard_normal(V) * 3.0 + np.repeat(rng.uniform(-2, 2, (V + 4095) // 4096), 4096)[:V]
        H = oracle.node_statistics(z[None], 1.0)["H"][0]
        assert abs(merged_entropy(z, 4096, batch=8) - H) < 1e-9
        assert abs(merged_entropy(z, 4096, batch=3) - H) < 1e-9


def test_near_threshold_case_properties():
    w = synth.workload("vicuna-7b", V=9000)
    tc = tree_case(w, seed=0)
    c = typical_threshold_case(w, tc, seed=0)
    t = tc["ref"]
    st = c["ref"]["stats"][0]
    parents = sorted({int(t["parent"][n]) for n in range(1, len(t["parent"]))})
    for n in parents:
        assert 0.3 * np.exp(-st["H"][n]) < 0.09          # the entropy branch binds
    ratios = []
    for ch in range(1, len(t["parent"])):
        n = int(t["parent"][ch])
        p = np.exp(st["z"][n, t["tree_candidates"][0, ch]] - st["m"][n]) / st["S"][n]
        ratios.append(p / st["thr"][n])
    r = np.array(ratios)
    assert np.all((np.abs(np.log(r)) >= np.log(1.04)) & (np.abs(np.log(r)) <= np.log(3.04)))
    assert c["flips"]["shift"] > 0 and c["changed"]["shift"]
