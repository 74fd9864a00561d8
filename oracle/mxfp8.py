"""MXFP8 quantization: backward re-quantization with stochastic rounding, and
round-to-nearest quantization of the output gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Inkling 2 Small uses four-bit training ...", ai-primer,
section "Stochastic rounding across transposes", and section "NVFP4 forward,
MXFP8 backward"): the backward pass dequantizes the saved forward weights and
activations, transposes them in higher precision, re-quantizes them to MXFP8
with stochastic rounding, and computes the gradients with MXFP8 matmuls.
MXFP8 costs 8.25 bits per value (section "Block scales and per-token
activations"): 8-bit elements plus one 8-bit scale per 32.

Readings taken where the pages are silent:

* Elements are E4M3FN; the shared scale is E8M0 over 32 consecutive elements
  of the transposed (contraction-contiguous) row.
* Block exponent: the smallest e with amax <= 448 * 2^e (``e8m0_ceil``), so no
  element saturates; y = v * 2^-e in float32.
* "Higher precision" for the transpose is float32 (dequantized values are
  float32).
* The stochastic rounding draw for the element at linear index idx of the
  output buffer [cols, P] is ``philox.uniform16(seed, tag, idx)``.
* The output gradient dY is quantized with round-to-nearest-even (the pages
  restrict stochastic rounding to the saved weights and activations).

Grouped layout: rows [offsets[g], offsets[g+1]) of the input (tokens of
expert g, or the N rows of expert g's weight) become output columns
[padded_offsets[g], padded_offsets[g] + len) of the output [cols, P]; the
columns up to the next multiple of 32 are zero, so every 32-block of the
output lies inside one group. Columns at or after padded_offsets[G] are not
part of the result (returned as zero here; the device leaves them untouched).
"""

import numpy as np

from . import formats as F
from . import nvfp4 as Q
from . import philox

MX_BLOCK = 32


def pad32(n):
    return (np.asarray(n, dtype=np.int64) + 31) // 32 * 32


def padded_offsets_from_offsets(offsets):
    """Exclusive scan of pad32(group length)."""
    off = np.asarray(offsets, dtype=np.int64)
    lens = np.diff(off)
    return np.concatenate([[0], np.cumsum(pad32(lens))]).astype(np.int64)


def transpose_grouped(v, offsets, padded_offsets, P):
    """float32 [rows, cols] -> float32 [cols, P], grouped and zero padded."""
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    out = np.zeros((cols, P), dtype=np.float32)
    off = np.asarray(offsets, dtype=np.int64)
    poff = np.asarray(padded_offsets, dtype=np.int64)
    for g in range(off.shape[0] - 1):
        a, b = int(off[g]), int(off[g + 1])
        p = int(poff[g])
        out[:, p:p + (b - a)] = v[a:b, :].T
    return out


def block_exponents(t):
    """E8M0 exponent per 32-block along the last axis of float32 t [R, C]."""
    R, C = t.shape
    amax = np.abs(t).reshape(R, C // MX_BLOCK, MX_BLOCK).max(axis=2)
    return F.e8m0_ceil_exponent(amax)


def _scaled(t, e):
    """y = t * 2^-e per 32-block, in float32 (exact except below 2^-126)."""
    R, C = t.shape
    f = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)
    y = t.reshape(R, C // MX_BLOCK, MX_BLOCK) * f[:, :, None]
    return y.astype(np.float32).reshape(R, C)


def quantize_rne(t):
    """float32 [R, C] (C % 32 == 0) -> (E4M3 codes [R, C], E8M0 [R, C/32])."""
    t = np.asarray(t, dtype=np.float32)
    e = block_exponents(t)
    y = _scaled(t, e)
    return F.e4m3_rne(y), (e + 127).astype(np.uint8)


def quantize_sr(t, seed, tag, idx_base=0):
    """float32 [R, C] -> MXFP8 with stochastic rounding; the draw for element
    (i, j) uses linear index idx_base + i*C + j."""
    t = np.asarray(t, dtype=np.float32)
    R, C = t.shape
    e = block_exponents(t)
    y = _scaled(t, e)
    u = philox.uniform16_range(seed, tag, idx_base, R * C).reshape(R, C)
    return F.e4m3_sr(y, u), (e + 127).astype(np.uint8)


def dequantize(e4m3, e8m0):
    """MXFP8 -> float64 values e4m3 * 2^(e8m0-127) (exact)."""
    q = F.e4m3_decode(np.asarray(e4m3))
    R, C = q.shape
    s = F.e8m0_decode(np.asarray(e8m0))
    return (q.reshape(R, C // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(R, C)


def requant_sr(codes, scales, outer, offsets, padded_offsets, P, seed, tag,
               rows_per_group=None):
    """Backward re-quantization of a saved NVFP4 tensor.

    NVFP4 [rows, cols] -> dequantize (float32) -> grouped transpose to
    [cols, P] -> MXFP8 with stochastic rounding. Returns (E4M3 [cols, P],
    E8M0 [cols, P/32]). rows_per_group: None for per-row outer scales
    (activations), N for per-expert outer scales of weights stored [E*N, K].
    """
    if P % MX_BLOCK:
        raise ValueError("P must be a multiple of 32")
    v = Q.dequantize(codes, scales, outer, rows_per_group=rows_per_group)
    t = transpose_grouped(v, offsets, padded_offsets, P)
    return quantize_sr(t, seed, tag)


def quantize_rowwise(x):
    """Output gradient [rows, cols] (float32 or bfloat16 bits) -> MXFP8 RNE
    with blocks of 32 along cols."""
    return quantize_rne(Q._as_f32(x))


def quantize_colwise_grouped(x, offsets, padded_offsets, P):
    """Output gradient [rows, cols] -> grouped transpose [cols, P] -> MXFP8 RNE."""
    t = transpose_grouped(Q._as_f32(x), offsets, padded_offsets, P)
    return quantize_rne(t)
