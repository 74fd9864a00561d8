"""NVFP4 backward: the gradient matmuls on NVFP4 operands re-quantized with
stochastic rounding, the alternative to the MXFP8 backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the lab's first experiments ran both passes in NVFP4 and were given up
("Inkling 2 Small uses four-bit training ...", ai-primer, section "NVFP4
forward, MXFP8 backward"), and a 4-bit backward is what the team says it is
exploring ("Thinking Machines details ... 4 bit", advanceintelligence.ai,
section "What to expect next"). The backward recipe the pages do give
(section "Stochastic rounding across transposes": dequantize the saved
tensors, transpose in higher precision, re-quantize with stochastic rounding,
run the gradient matmuls) is kept, with NVFP4 instead of MXFP8 as the target.

Readings (none of this is on the pages):
* Element rounding is stochastic everywhere in this backward, the output
  gradient included (a 4-bit round-to-nearest gradient is biased, which is
  what the recipe's stochastic rounding is there to avoid). The draw for the
  element at linear index idx of an output buffer is
  ``philox.uniform16(seed, tag, idx)``; tags 5 = activations, 6 = weights,
  7 = dY row-wise, 8 = dY transposed.
* Block scales are rounded up to the next E4M3 value,
  S = E4M3_ceil(bmax / (6 s)), so every scaled element lies in [-6, 6] and
  stochastic rounding never has to saturate (the MXFP8 path's exponent is
  chosen by the same principle). Only float32 rounding of the scaled value
  can land a few units in the last place above 6; such a value becomes 6.
* Outer scales: dY row-wise keeps one per token, as the forward activations;
  an operand whose contraction runs over tokens (the transposed activations
  and the transposed dY) cannot, and takes one per expert group, the
  granularity the pages give the weights; the transposed weights keep one per
  expert. s = A / 2688 with A the maximum magnitude it covers, as forward.
* Layouts: transposed activations and dY are [cols, P] with group g in
  columns [padded_offsets[g], padded_offsets[g+1]) and zeros after its rows;
  here the segments are padded to 128 (the gradient kernel's contraction
  step) instead of 32. Transposed weights are stored per expert, [E, K, N]
  (expert e's W_e transposed), so that dgrad is the forward grouped GEMM.
* dgrad[r, k]  = s_dy[r] s_w[g] sum_n dY4[r, n] WT4[g, k, n]
  wgrad[g,n,k] = s_dyT[g] s_xT[g] sum over g's columns p of dYT4[n, p] XT4[k, p]
"""

import numpy as np

from . import formats as F
from . import gemm as G
from . import mxfp8 as MX
from . import nvfp4 as Q
from . import philox

TAG_X, TAG_W, TAG_DY_ROW, TAG_DY_COL = 5, 6, 7, 8
ALIGN = 128
OUTER_DIVISOR = np.float32(6.0 * 448.0)


def padded_offsets(offsets, align=ALIGN):
    """Exclusive scan of the group lengths rounded up to ``align``."""
    off = np.asarray(offsets, dtype=np.int64)
    lens = np.diff(off)
    return np.concatenate([[0], np.cumsum((lens + align - 1) // align * align)]).astype(np.int64)


def e4m3_ceil(t):
    """Smallest E4M3 magnitude >= t (t >= 0), 448 for larger t -> code."""
    t = np.asarray(t, dtype=np.float64)
    grid = F.E4M3_GRID
    idx = np.searchsorted(grid, t, side="left")
    return np.minimum(idx, grid.shape[0] - 1).astype(np.uint8)


def e2m1_sr_sat(y, u16):
    """Stochastic rounding onto E2M1; magnitudes above 6 become 6."""
    y = np.asarray(y, dtype=np.float64)
    six = np.where(np.signbit(y), -6.0, 6.0)
    ys = np.where(np.abs(y) > 6.0, six, y)
    return F.e2m1_sr(ys, u16)


def _quantize_blocks_sr(t, s, seed, tag, idx0=0):
    """t float32 [R, C] with outer scale s float32 [R] per row -> (codes
    [R, C/2], scales [R, C/16]); draws at linear index idx0 + r*C + c."""
    t = np.asarray(t, dtype=np.float32)
    R, C = t.shape
    nb = C // Q.BLOCK
    tb = t.reshape(R, nb, Q.BLOCK)
    bmax = np.abs(tb).max(axis=2)
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        d = (np.float32(6.0) * s).astype(np.float32)
        q = (bmax / d[:, None]).astype(np.float32)
        q = np.where((s == 0)[:, None], np.float32(0), q)
        sc = e4m3_ceil(q)
        S = F.e4m3_decode(sc).astype(np.float32)
        r = (np.float32(1.0) / (S * s[:, None]).astype(np.float32)).astype(np.float32)
        y = (tb * r[:, :, None]).astype(np.float32)
    u = philox.uniform16_range(seed, tag, idx0, R * C).reshape(R, nb, Q.BLOCK)
    y = np.where((sc == 0)[:, :, None], np.float32(0), y)     # zero blocks (no division)
    codes = e2m1_sr_sat(y, u)
    signed_zero = (np.signbit(tb).astype(np.uint8) << 3)
    codes = np.where((sc == 0)[:, :, None], signed_zero, codes).astype(np.uint8)
    return Q.pack_codes(codes.reshape(R, C)), sc


def quantize_sr_rows(x, seed, tag=TAG_DY_ROW):
    """Row-wise NVFP4 with stochastic rounding, one outer scale per row:
    (codes [R, C/2], scales [R, C/16], outer [R])."""
    x = Q._as_f32(x)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (amax / OUTER_DIVISOR).astype(np.float32)
    c, sc = _quantize_blocks_sr(x, s, seed, tag)
    return c, sc, s


def quantize_sr_grouped_T(v, offsets, padded, P, seed, tag):
    """v float32 [rows, cols] (rows grouped by ``offsets``) -> grouped
    transpose [cols, P] -> NVFP4 with stochastic rounding, one outer scale per
    group: (codes [cols, P/2], scales [cols, P/16], outer [G])."""
    v = np.asarray(v, dtype=np.float32)
    off = np.asarray(offsets, dtype=np.int64)
    poff = np.asarray(padded, dtype=np.int64)
    Gn = off.shape[0] - 1
    t = MX.transpose_grouped(v, off, poff, P)
    cols = t.shape[0]
    amax = np.array([np.abs(v[off[g]:off[g + 1]]).max() if off[g + 1] > off[g] else 0.0
                     for g in range(Gn)], dtype=np.float32)
    sg = (amax / OUTER_DIVISOR).astype(np.float32)
    codes = np.zeros((cols, P // 2), np.uint8)
    scales = np.zeros((cols, P // 16), np.uint8)
    for g in range(Gn):
        a, b = int(poff[g]), int(poff[g + 1])
        if b == a:
            continue
        seg = np.ascontiguousarray(t[:, a:b])
        # draws by the output's linear index k * P + p: row by row
        for k in range(cols):
            c, sc = _quantize_blocks_sr(seg[k:k + 1], sg[g:g + 1], seed, tag, idx0=k * P + a)
            codes[k, a // 2:b // 2] = c[0]
            scales[k, a // 16:b // 16] = sc[0]
    return codes, scales, sg


def requant_sr(codes, scales, outer, offsets, padded, P, seed, tag=TAG_X):
    """Saved per-row NVFP4 activations [rows, cols] -> dequantize (float32) ->
    grouped transpose -> NVFP4 with stochastic rounding, outer per group."""
    v = Q.dequantize(codes, scales, outer)
    return quantize_sr_grouped_T(v, offsets, padded, P, seed, tag)


def requant_weights_sr(codes, scales, outer, E, seed, tag=TAG_W):
    """Saved weights NVFP4 [E*N, K] (outer per expert) -> per expert
    transpose -> NVFP4 [E*K, N] with stochastic rounding, outer per expert;
    draws at the linear index (e*K + k)*N + n of that layout."""
    Nn = np.asarray(codes).shape[0] // E
    v = Q.dequantize(codes, scales, outer, rows_per_group=Nn)       # [E*N, K]
    K = v.shape[1]
    vt = v.reshape(E, Nn, K).transpose(0, 2, 1).reshape(E * K, Nn)  # [E*K, N]
    amax = np.abs(v.reshape(E, Nn * K)).max(axis=1).astype(np.float32)
    s = (amax / OUTER_DIVISOR).astype(np.float32)
    c, sc = _quantize_blocks_sr(vt, np.repeat(s, K), seed, tag)
    return c, sc, s


def dgrad(dy_q, wT_q, offsets, K, accum="fp32"):
    """dX [M, K] from dY NVFP4 [M, N] (outer per row) and the per-expert
    transposed weights [E*K, N] (outer per expert): the forward grouped GEMM."""
    return G.fwd_grouped(*dy_q, *wT_q, offsets, K, accum=accum)


def wgrad(dyT_q, xT_q, padded, accum="fp32"):
    """dW [G, N, K] from dYT NVFP4 [N, P] and XT NVFP4 [K, P], one outer
    scale per group each."""
    dyc, dys, dyo = dyT_q
    xc, xs, xo = xT_q
    A = Q.dequantize(dyc, dys, None, apply_outer=False)            # [N, P], exact
    B = Q.dequantize(xc, xs, None, apply_outer=False)              # [K, P]
    poff = np.asarray(padded, dtype=np.int64)
    Gn = poff.shape[0] - 1
    dt = np.float64 if accum == "fp64" else np.float32
    out = np.zeros((Gn, A.shape[0], B.shape[0]), dtype=dt)
    for g in range(Gn):
        a, b = int(poff[g]), int(poff[g + 1])
        if b == a:
            continue
        acc = G._mm(A[:, a:b], B[:, a:b].T, accum)
        out[g] = ((acc * dt(dyo[g])).astype(dt) * dt(xo[g])).astype(dt)
    return out
