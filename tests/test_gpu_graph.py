"""The whole expert-layer step captured in a HIP graph (the way the benchmark
times it) gives the eager step's results on every replay, with eager work and
synchronizations between the replays. The step clears its counters with
kernels, not memset nodes, so replays after the first stay correct."""

import numpy as np
import pytest

from helpers import ensure_built
from workloads import gen

pytestmark = pytest.mark.gpu


def test_layer_step_graph_replays_match_eager():
    ensure_built()
    import torch
    from precision_moe_numerics_nvfp4_amd.layer import ExpertLayerStep
    T, K, N, E, k = 600, 256, 512, 4, 2
    def inputs(seed):
        w = gen.small_moe(T=T, K=K, N=N, E=E, k=k, cfg=20 + seed)
        dy = gen.backward_dy(T * k, N, cfg=20 + seed)
        dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
                         if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))).cuda()
        return dev(w["x"]), dev(w["w"]), dev(w["topk"]), dev(dy)
    a_in, b_in = inputs(0), inputs(1)
    L = ExpertLayerStep(T, K, N, E, k, out_dtype=torch.bfloat16)
    outs = lambda: (L.y, L.dx, L.dw, L.xT[0], L.xT[1], L.wT[0], L.dyT[0], L.perm["offsets"])
    L.step(*a_in)
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in outs()]
    L.step(*b_in)
    torch.cuda.synchronize()
    ref_b = [t.clone() for t in outs()]
    assert not all(torch.equal(x, y) for x, y in zip(ref_a, ref_b))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.step(*a_in)
    for rep in range(3):
        L.step(*b_in)                                  # eager work between replays
        torch.cuda.synchronize()
        for x, y in zip(ref_b, outs()):
            assert torch.equal(x, y), f"eager step after replay {rep}"
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(ref_a, outs())):
            assert torch.equal(x, y), f"replay {rep}, output {i}"
