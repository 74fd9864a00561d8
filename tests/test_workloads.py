"""The seeded workload generators reproduce the stated recipes (CPU only)."""

import numpy as np

from workloads import gen


def test_generators_are_seeded_and_shaped():
    a = gen.small_moe(T=64, K=32, N=16, E=8, k=2)
    b = gen.small_moe(T=64, K=32, N=16, E=8, k=2)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["topk"], b["topk"])
    assert a["x"].dtype == np.uint16 and a["w"].shape == (8 * 16, 32)
    t = a["topk"]
    assert all(len(set(row)) == 2 for row in t) and t.min() >= 0 and t.max() < 8


def test_zipf_placement_and_local_share():
    ids = gen.zipf_placement()
    assert sorted(ids) == list(range(384))
    assert ids[0] == 0 and ids[1] == 48 and ids[8] == 1          # round-robin deal
    topk = gen.route_zipf(3, 32768, k=8)
    assert all(len(set(r)) == 8 for r in topk[:2000])
    local = (topk >= 144) & (topk < 192)
    share = local.mean()
    assert 0.10 < share < 0.14                                   # about one eighth
    counts = np.bincount(topk[local] - 144, minlength=48)
    assert counts.max() > 20 * counts.min()                      # Zipf skew


def test_single_expert_outliers():
    w = gen.single_expert()
    assert w["x"].shape == (64, 256) and w["w"].shape == (512, 256)
    assert np.abs(w["x"]).max() > 20 and np.abs(w["w"]).max() > 20
