"""The three grouped matmuls of the expert layer, on already-quantized operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the forward expert-layer matmuls run in NVFP4 and the gradient matmuls
in MXFP8 ("Inkling 2 Small uses four-bit training ...", ai-primer, section
"NVFP4 forward, MXFP8 backward"; section "Stochastic rounding across
transposes", last step). Each result is the plain definition: dequantize both
operands exactly (every NVFP4 element times its block scale, every MXFP8
element times its power of two, is exact in float32), contract, then apply
the outer scales. ``accum`` selects float32 accumulation (numpy's float32
matmul) or float64; both are the same mathematical sum and differ only by
rounding.

Shapes (M = routed rows, G = groups/experts, row-major):
* forward:  Y[r, n]    = s_x[r] * s_w[g] * sum_k A[r, k] * B[g, n, k]
            A = X_perm NVFP4 [M, K], B = W NVFP4 stored [G, N, K]
* dgrad:    dX[r, k]   = sum_n dY8[r, n] * W8[k, g*N + n]
            dY8 MXFP8 [M, N] (blocks along n), W8 MXFP8 [K, G*N]
* wgrad:    dW[g, n, k] = sum_p dYT8[n, p] * XT8[k, p] over p in group g's
            padded column segment; dYT8 [N, P], XT8 [K, P]
* forward, all MXFP8 (the full-MXFP8 reference the NVFP4 forward is compared
  against: page 2, TL;DR and section "Expert precision and convolution
  caches"):
            Y[r, n]     = sum_k X8[r, k] * W8[g, n, k]
            X8 MXFP8 [M, K] (blocks along k), W8 MXFP8 stored [G, N, K]
Rows r of group g are offsets[g] <= r < offsets[g+1].
"""

import numpy as np

from . import nvfp4 as Q
from . import mxfp8 as MX


def _mm(a, b, accum):
    if accum == "fp64":
        return a.astype(np.float64) @ b.astype(np.float64)
    return (a.astype(np.float32) @ b.astype(np.float32)).astype(np.float32)


def fwd_grouped(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, offsets,
                N, accum="fp32"):
    """NVFP4 forward grouped GEMM -> float32 [M, N] (float64 if accum='fp64')."""
    A = Q.dequantize(a_codes, a_scales, None, apply_outer=False)
    G = int(np.asarray(b_outer).shape[0])
    K = A.shape[1]
    B = Q.dequantize(np.asarray(b_codes).reshape(G * N, K // 2),
                     np.asarray(b_scales).reshape(G * N, K // 16),
                     None, apply_outer=False).reshape(G, N, K)
    off = np.asarray(offsets, dtype=np.int64)
    M = int(off[-1])
    dt = np.float64 if accum == "fp64" else np.float32
    Y = np.zeros((M, N), dtype=dt)
    sx = np.asarray(a_outer, dtype=dt)
    sw = np.asarray(b_outer, dtype=dt)
    for g in range(G):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        acc = _mm(A[a:b], B[g].T, accum)
        Y[a:b] = ((acc * sx[a:b, None]).astype(dt) * sw[g]).astype(dt)
    return Y


def dgrad_grouped(dy_e4m3, dy_e8m0, w_e4m3, w_e8m0, offsets, N, accum="fp32"):
    """MXFP8 dgrad grouped GEMM -> [M, K]."""
    dY = MX.dequantize(dy_e4m3, dy_e8m0)          # [M, N]
    W = MX.dequantize(w_e4m3, w_e8m0)             # [K, G*N]
    off = np.asarray(offsets, dtype=np.int64)
    M = int(off[-1])
    K = W.shape[0]
    dt = np.float64 if accum == "fp64" else np.float32
    out = np.zeros((M, K), dtype=dt)
    for g in range(off.shape[0] - 1):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        out[a:b] = _mm(dY[a:b], W[:, g * N:(g + 1) * N].T, accum)
    return out


def fwd_grouped_mxfp8(x_e4m3, x_e8m0, w_e4m3, w_e8m0, offsets, N, accum="fp32"):
    """All-MXFP8 forward grouped GEMM -> [M, N]; weights [G*N, K] or [G, N, K]."""
    X = MX.dequantize(x_e4m3, x_e8m0)             # [M, K]
    K = X.shape[1]
    off = np.asarray(offsets, dtype=np.int64)
    G = off.shape[0] - 1
    W = MX.dequantize(np.asarray(w_e4m3).reshape(G * N, K),
                      np.asarray(w_e8m0).reshape(G * N, K // 32)).reshape(G, N, K)
    M = int(off[-1])
    dt = np.float64 if accum == "fp64" else np.float32
    out = np.zeros((M, N), dtype=dt)
    for g in range(G):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        out[a:b] = _mm(X[a:b], W[g].T, accum)
    return out


def wgrad_grouped(dyT_e4m3, dyT_e8m0, xT_e4m3, xT_e8m0, padded_offsets,
                  accum="fp32"):
    """MXFP8 wgrad grouped GEMM -> [G, N, K]."""
    dYT = MX.dequantize(dyT_e4m3, dyT_e8m0)       # [N, P]
    XT = MX.dequantize(xT_e4m3, xT_e8m0)          # [K, P]
    poff = np.asarray(padded_offsets, dtype=np.int64)
    G = poff.shape[0] - 1
    N, K = dYT.shape[0], XT.shape[0]
    dt = np.float64 if accum == "fp64" else np.float32
    out = np.zeros((G, N, K), dtype=dt)
    for g in range(G):
        a, b = int(poff[g]), int(poff[g + 1])
        if b == a:
            continue
        out[g] = _mm(dYT[:, a:b], XT[:, a:b].T, accum)
    return out
