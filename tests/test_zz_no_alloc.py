"""The permute entry point that allocates nothing (moe_permute_noalloc: the
count table in the library's own per-GPU array) against moe_permute (the
caller's workspace), through the C ABI: the same bytes on calls in a row,
each later call smaller than the one before (the array keeps the previous
call's contents), across the three-launch and one-launch forms; and the size
limit rejected on the host."""

import numpy as np
import pytest

from helpers import ensure_built, from_dev, to_dev
from oracle import nvfp4 as Q
from workloads import gen

EWORKSPACE = 3


def _fresh_out(torch, T, k, n_local, K):
    dev = "cuda"
    cap = T * k
    return {"offsets": torch.full((n_local + 1,), -7, dtype=torch.int64, device=dev),
            "padded_offsets": torch.full((n_local + 1,), -7, dtype=torch.int64, device=dev),
            "row_token": torch.full((cap,), -7, dtype=torch.int32, device=dev),
            "row_slot": torch.full((cap,), -7, dtype=torch.int32, device=dev),
            "pair_row": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "codes": torch.zeros((cap, K // 2), dtype=torch.uint8, device=dev),
            "scales": torch.zeros((cap, K // 16), dtype=torch.uint8, device=dev),
            "outer": torch.zeros((cap,), dtype=torch.float32, device=dev)}


@pytest.mark.gpu
def test_permute_noalloc_matches_permute():
    ensure_built()
    import torch
    import precision_moe_numerics_nvfp4_amd as nv
    assert torch.cuda.is_available()
    K = 256
    # pairs: 32768 and 17600 (three-launch form, smaller table the second
    # time), then 8000 (one-launch form), then 20000 over 4 experts
    cases = [(4096, 8, 144, 48, 601), (2200, 8, 144, 48, 602), (1000, 8, 144, 48, 603),
             (5000, 4, 0, 4, 604)]
    for T, k, e0, nl, seed in cases:
        print(f"[noalloc] T={T} k={k} e0={e0} n_local={nl}", flush=True)
        if nl == 48:
            topk = gen.route_zipf(seed, T, k=k)
        else:
            topk = gen.route_uniform(seed, T, 6, k)
        x = gen.to_bf16_bits(gen.normal(seed, 0, (T, K)))
        xq = tuple(to_dev(a) for a in Q.quantize(x))
        t_d = to_dev(topk)
        ref = nv.moe_permute(t_d, e0, nl, *xq)
        got = nv.moe_permute_noalloc(t_d, e0, nl, *xq, out=_fresh_out(torch, T, k, nl, K))
        torch.cuda.synchronize()
        M = int(from_dev(ref["offsets"])[-1])
        for name in ("offsets", "padded_offsets", "pair_row"):
            assert np.array_equal(from_dev(got[name]), from_dev(ref[name])), name
        for name in ("row_token", "row_slot", "codes", "scales", "outer"):
            assert np.array_equal(from_dev(got[name])[:M].view(np.uint8),
                                  from_dev(ref[name])[:M].view(np.uint8)), name


def test_permute_noalloc_rejects_oversized_tables():
    """More than 4 MiB of count table is refused before any HIP call."""
    ensure_built()
    import ctypes
    from precision_moe_numerics_nvfp4_amd import binding
    L = binding.lib()
    fake = ctypes.c_void_p(0x10000)
    T, k, nl = 300000, 1, 1024                     # 1172 chunks x 1024 experts x 4 B > 4 MiB
    assert L.nvfp4moe_permute_workspace_size(T, k, nl) > 4 << 20
    args = (fake, T, k, 0, nl, fake, fake, fake, 256, fake, fake, fake, fake, None, fake, fake,
            fake, None)
    assert L.moe_permute_noalloc(*args) == EWORKSPACE
    T = 261888                                     # 1023 chunks: fits
    assert L.nvfp4moe_permute_workspace_size(T, k, nl) <= 4 << 20
