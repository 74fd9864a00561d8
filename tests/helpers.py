"""Shared test helpers: host<->device marshalling and oracle pipelines.

The oracle is called on the same host arrays that are uploaded to the GPU.
"""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    """Build the HIP library if it is not there yet (tests load what is built)."""
    from precision_moe_numerics_nvfp4_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        subprocess.run([sys.executable, "-m", "precision_moe_numerics_nvfp4_amd.build"],
                       cwd=ROOT, check=True)
    return binding.LIB_PATH


def to_dev(a):
    """numpy -> GPU tensor; uint16 arrays are bfloat16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def from_dev(t):
    """GPU tensor -> numpy; bfloat16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_gemm_close(y, ref64, groups, absbound=None, tol=1e-3, what="gemm", elementwise=True):
    """Per group: max|y - ref| <= tol * max|ref| (the contract); with
    `elementwise`, relative error <= tol where |ref| >= 1e-2 max|ref|; and,
    when given, |y - ref| <= absbound elementwise (a summation error bound)."""
    y = np.asarray(y, dtype=np.float64)
    for (a, b) in groups:
        if b <= a:
            continue
        r = ref64[a:b]
        d = np.abs(y[a:b] - r)
        m = np.abs(r).max()
        assert d.max() <= tol * m + 1e-30, f"{what}: group [{a},{b}) normwise {d.max() / max(m, 1e-300):.3e}"
        big = np.abs(r) >= 1e-2 * m
        if elementwise and big.any():
            rel = (d[big] / np.abs(r[big])).max()
            assert rel <= tol, f"{what}: group [{a},{b}) elementwise {rel:.3e}"
        if absbound is not None:
            viol = d > absbound[a:b] * 1.0000001 + 1e-37
            assert not viol.any(), f"{what}: {viol.sum()} elements exceed the summation error bound"


def w8_blocked(a, G):
    """A re-quantized weight in the oracle's [K, G*N] arrangement (or its
    E8M0 bytes [K, G*N/32]) -> the library's per-expert blocks [G*K, N]."""
    a = np.asarray(a)
    K, GN = a.shape
    return np.ascontiguousarray(a.reshape(K, G, GN // G).transpose(1, 0, 2)).reshape(G * K, GN // G)


def w8_tokenwise(a, G):
    """The inverse of w8_blocked: [G*K, N] -> [K, G*N]."""
    a = np.asarray(a)
    GK, N = a.shape
    return np.ascontiguousarray(a.reshape(G, GK // G, N).transpose(1, 0, 2)).reshape(GK // G, G * N)


def worst_elementwise(y, ref64, groups, floor=1e-2):
    """Largest |y - ref| / |ref| over elements with |ref| >= floor * (the
    group's max |ref|): the elementwise error a normwise contract allows."""
    y = np.asarray(y, dtype=np.float64)
    worst = 0.0
    for (a, b) in groups:
        if b <= a:
            continue
        r = ref64[a:b]
        m = np.abs(r).max()
        big = np.abs(r) >= floor * m
        if big.any():
            worst = max(worst, float((np.abs(y[a:b] - r)[big] / np.abs(r[big])).max()))
    return worst


def sr_mean_sd(v, e8):
    """Analytic standard deviation of mean(SR(v)) - mean(v) for float values
    v [R, C] re-quantized to E4M3 with E8M0 block exponents e8 [R, C/32]:
    each element rounds up with probability D over a gap g, so its variance
    is D (1 - D) g^2."""
    from oracle import formats as F
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    s = np.exp2(np.repeat(np.asarray(e8, dtype=np.float64) - 127, 32, axis=1))
    a = np.abs(v) / s
    lo_i = np.searchsorted(F.E4M3_GRID, a, side="right") - 1
    at_max = lo_i >= 126
    hi = F.E4M3_GRID[np.minimum(lo_i + 1, 126)]
    gap = np.where(at_max, 1.0, hi - F.E4M3_GRID[lo_i])
    D = (a - F.E4M3_GRID[lo_i]) / gap
    var = np.where(at_max, 0.0, D * (1 - D)) * (gap * s) ** 2
    return np.sqrt(var.sum()) / v.size
