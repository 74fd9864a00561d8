"""NVFP4 quantization (per token / per expert outer scale) and dequantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Inkling 2 Small uses four-bit training ...", ai-primer,
section "Block scales and per-token activations"): 4-bit values, one E4M3
scale per block of 16 consecutive values, and an additional FP32 outer scale;
one outer scale per expert for weights and one per token for activations (so a
token's quantization depends on no other token).

What they leave open, and the reading taken (all arithmetic is IEEE binary32
with round-to-nearest-even and no fused multiply-add, in this order):

  1. A = max |x| over the outer-scale group (a row, or a whole expert).
  2. A == 0: outer scale 0, every block scale 0, every code a signed zero.
  3. s = A / 2688, where 2688 = 6 * 448 maps A onto the top of both the E2M1
     grid (6) and the E4M3 grid (448); d = 6 * s.
  4. Block b of 16: S_b = E4M3_RNE_saturating(max|x_b| / d).
  5. S_b == 0: the block's codes are signed zeros.
  6. Otherwise r_b = 1 / (S_b * s) (the product rounded, then a correctly
     rounded reciprocal) and each code is E2M1_RNE_saturating(x * r_b).

The outer scale stored is s. Dequantized value: v = (e2m1 * S_b) * s, where
the inner product is exact and only the multiplication by s rounds.

Layouts: codes uint8 [rows, cols/2] with element 2j in bits 3..0 and element
2j+1 in bits 7..4; scales uint8 [rows, cols/16]; outer float32 [rows] (per
row) or [rows / rows_per_group] (per group). cols must be a multiple of 16.
"""

import numpy as np

from . import formats as F

OUTER_DIVISOR = np.float32(2688.0)      # 6 * 448
BLOCK = 16


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:            # bfloat16 bit patterns
        return F.bf16_bits_to_f32(x)
    return x.astype(np.float32)


def pack_codes(codes):
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, even element low."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_codes(packed):
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize(x, rows_per_group=None):
    """NVFP4-quantize x [rows, cols] (float32 or bfloat16 bits as uint16).

    rows_per_group None: one outer scale per row (activations, one per
    token). Otherwise rows_per_group consecutive rows share one outer scale
    (weights stored [E*N, K] with rows_per_group = N: one per expert).

    Returns (codes [rows, cols/2] uint8, scales [rows, cols/16] uint8,
    outer float32 [rows] or [rows/rows_per_group]).
    """
    x = _as_f32(x)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 16")
    ax = np.abs(x)

    # step 1: amax per outer-scale group
    if rows_per_group is None:
        amax = ax.max(axis=1) if cols else np.zeros(rows, np.float32)
        per_row_amax = amax
    else:
        if rows % rows_per_group:
            raise ValueError("rows must be a multiple of rows_per_group")
        g = rows // rows_per_group
        amax = ax.reshape(g, rows_per_group * cols).max(axis=1)
        per_row_amax = np.repeat(amax, rows_per_group)

    # step 3: outer scale
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s_out = (amax / OUTER_DIVISOR).astype(np.float32)
        s = (per_row_amax / OUTER_DIVISOR).astype(np.float32)
        d = (np.float32(6.0) * s).astype(np.float32)

        # step 4: block scales
        nb = cols // BLOCK
        xb = x.reshape(rows, nb, BLOCK)
        ab = ax.reshape(rows, nb, BLOCK).max(axis=2)
        t = (ab / d[:, None]).astype(np.float32)
        t = np.where(per_row_amax[:, None] == 0, np.float32(0), t)
        scale_codes = F.e4m3_rne(t)
        S = F.e4m3_decode(scale_codes).astype(np.float32)

        # step 6: codes
        r = (np.float32(1.0) / (S * s[:, None]).astype(np.float32)).astype(np.float32)
        y = (xb * r[:, :, None]).astype(np.float32)
        codes = F.e2m1_rne(y)

    # steps 2 and 5: zero blocks give signed zeros
    zero_block = (scale_codes == 0)[:, :, None]
    signed_zero = (np.signbit(xb).astype(np.uint8) << 3)
    codes = np.where(zero_block, signed_zero, codes).astype(np.uint8)
    codes = codes.reshape(rows, cols)
    return pack_codes(codes), scale_codes.astype(np.uint8), s_out


def dequantize(codes, scales, outer, rows_per_group=None, apply_outer=True):
    """NVFP4 -> float32: v = (e2m1 * S) * s with one rounding (the last).

    With apply_outer=False returns e2m1 * S (exact in float32).
    """
    c = unpack_codes(codes)
    rows, cols = c.shape
    S = F.e4m3_decode(np.asarray(scales)).astype(np.float64)
    inner = F.e2m1_decode(c).reshape(rows, cols // BLOCK, BLOCK) * S[:, :, None]
    inner = inner.reshape(rows, cols).astype(np.float32)           # exact
    if not apply_outer:
        return inner
    s = np.asarray(outer, dtype=np.float32)
    if rows_per_group is not None:
        s = np.repeat(s, rows_per_group)
    return (inner * s[:, None]).astype(np.float32)


# ---------------------------------------------------------------- 16x16 tiles
#
# The alternative the pages report trying and rejecting ("Inkling 2 Small uses
# four-bit training ...", ai-primer, section "Stochastic rounding across
# transposes"): one scale shared by each 16x16 tile, so that a tensor and its
# transpose are represented by the same values; rejected as too sensitive to
# outliers (one large value pushes the rest of its tile to zero). Reading:
# the same two-level recipe as above with the 16-element block replaced by
# the 16x16 tile and the outer scale taken per group of rows (the expert for
# weights; one group for a whole tensor):
#   A = max|x| over the group, s = A / 2688, d = 6 s,
#   S_t = E4M3_RNE_saturating(max|x_t| / d) over tile t,
#   codes E2M1_RNE_saturating(x * (1 / (S_t * s))), signed zeros when S_t = 0.
# Layouts: codes as above; scales uint8 [rows/16, cols/16]; outer [groups].

TILE = 16


def quantize_tile16(x, rows_per_group=None):
    """16x16-tile NVFP4 of x [rows, cols] (rows and cols multiples of 16).

    rows_per_group None: one outer scale for the whole tensor; otherwise one
    per group of rows_per_group rows (a multiple of 16).
    Returns (codes [rows, cols/2], scales [rows/16, cols/16], outer [groups]).
    """
    x = _as_f32(x)
    rows, cols = x.shape
    if rows % TILE or cols % TILE:
        raise ValueError("rows and cols must be multiples of 16")
    rpg = rows if rows_per_group is None else rows_per_group
    if rpg % TILE or (rows and rows % rpg):
        raise ValueError("rows_per_group must be a multiple of 16 dividing rows")
    ax = np.abs(x)
    g = rows // rpg if rows else 0
    amax = ax.reshape(g, rpg * cols).max(axis=1) if g else np.zeros(0, np.float32)
    per_row_amax = np.repeat(amax, rpg)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s_out = (amax / OUTER_DIVISOR).astype(np.float32)
        s = (per_row_amax / OUTER_DIVISOR).astype(np.float32)
        d = (np.float32(6.0) * s).astype(np.float32)
        tr, tc = rows // TILE, cols // TILE
        at = ax.reshape(tr, TILE, tc, TILE).max(axis=(1, 3))              # [tr, tc]
        dt = d.reshape(tr, TILE)[:, 0]                                     # one d per tile row
        t = (at / dt[:, None]).astype(np.float32)
        t = np.where(per_row_amax.reshape(tr, TILE)[:, :1] == 0, np.float32(0), t)
        scale_codes = F.e4m3_rne(t)
        S = F.e4m3_decode(scale_codes).astype(np.float32)                  # [tr, tc]
        st = s.reshape(tr, TILE)[:, 0]
        r = (np.float32(1.0) / (S * st[:, None]).astype(np.float32)).astype(np.float32)
        rr = np.repeat(np.repeat(r, TILE, axis=0), TILE, axis=1)           # [rows, cols]
        y = (x * rr).astype(np.float32)
        codes = F.e2m1_rne(y)
    zero = np.repeat(np.repeat(scale_codes == 0, TILE, axis=0), TILE, axis=1)
    signed_zero = (np.signbit(x).astype(np.uint8) << 3)
    codes = np.where(zero, signed_zero, codes).astype(np.uint8)
    return pack_codes(codes), scale_codes.astype(np.uint8), s_out


def dequantize_tile16(codes, scales, outer, rows_per_group=None, apply_outer=True):
    """16x16-tile NVFP4 -> float32: v = (e2m1 * S_t) * s, one rounding."""
    c = unpack_codes(codes)
    rows, cols = c.shape
    S = F.e4m3_decode(np.asarray(scales)).astype(np.float64)
    Sx = np.repeat(np.repeat(S, TILE, axis=0), TILE, axis=1)
    inner = (F.e2m1_decode(c) * Sx).astype(np.float32)                     # exact
    if not apply_outer:
        return inner
    rpg = rows if rows_per_group is None else rows_per_group
    s = np.repeat(np.asarray(outer, dtype=np.float32), rpg)
    return (inner * s[:, None]).astype(np.float32)
