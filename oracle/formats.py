"""Element and scale formats, round-to-nearest-even and stochastic rounding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but do not define them bit by bit:
"Inkling 2 Small uses four-bit training ..." (ai-primer), section "Block scales
and per-token activations" gives NVFP4 as 4-bit values sharing an 8-bit E4M3
scale per 16 and MXFP8 at 8.25 bits/value; section "Stochastic rounding across
transposes" gives the FP4 worked example on neighbouring grid values 4 and 6.
The bit layouts below are the standard ones those names refer to:

* E2M1 (FP4): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf/NaN.
* E4M3 (OCP "E4M3FN"): sign bit 7, exponent bits 6..3 (bias 7), mantissa
  bits 2..0; exponent field 0 is subnormal (m * 2^-9); 0x7F/0xFF are NaN;
  largest finite magnitude 448 (0x7E).
* E8M0: an unsigned power of two 2^(c-127); 0xFF is NaN.

All values are produced in float64, where every grid value and every
product of an E2M1 value with an E4M3 scale is exact.
"""

import numpy as np

# ---------------------------------------------------------------- decoding

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (low nibble of each uint8); keeps -0."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c >> 3) & 1, -mag, mag)


def e4m3_decode(codes):
    """Value of 8-bit OCP E4M3FN codes, NaN for 0x7F and 0xFF; keeps -0."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = c & 7
    sub = m.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c >> 7, -mag, mag)


def e8m0_decode(codes):
    """Value 2^(c-127) of 8-bit E8M0 codes, NaN for 0xFF."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    v = np.power(2.0, c - 127)
    return np.where(c == 0xFF, np.nan, v)


# Non-negative magnitudes of each grid, indexed by magnitude code. For both
# grids "even code" == "mantissa LSB is 0" == even index.
E2M1_GRID = E2M1_MAGNITUDES.copy()                      # codes 0..7
E4M3_GRID = e4m3_decode(np.arange(0, 0x7F))             # codes 0..126, max 448
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def _sign_bit(y):
    """Sign bit of float values, including the sign of zero."""
    return np.signbit(np.asarray(y)).astype(np.int64)


# ---------------------------------------------------------------- rounding

def rne_to_grid(y, grid):
    """Round |y| to the nearest magnitude of ``grid``; ties go to the even
    index; magnitudes above the grid maximum saturate to it.

    Returns the magnitude index (an int64 array). Inputs must be finite.
    The comparison against the midpoint of two neighbours is exact in
    float64 for any float32 input.
    """
    a = np.abs(np.asarray(y, dtype=np.float64))
    n = grid.shape[0]
    lo = np.searchsorted(grid, a, side="right") - 1          # grid[lo] <= a
    lo = np.clip(lo, 0, n - 1)
    hi = np.minimum(lo + 1, n - 1)
    mid = (grid[lo] + grid[hi]) * 0.5
    up = (a > mid) | ((a == mid) & (lo % 2 == 1))
    idx = np.where(up, hi, lo)
    return np.where(a >= grid[-1], n - 1, idx)


def e2m1_rne(y):
    """float -> E2M1 code with round-to-nearest-even and saturation at 6.

    The sign bit of the code is the sign bit of ``y`` (so -0 and negative
    values that round to zero give code 0x8). The pages are silent on the
    rounding of forward-pass codes; round-to-nearest is their illustration
    of ordinary rounding ("Thinking Machines Lab ... 4-bit precision",
    section "Why Fewer Bits Means Faster Training": 3.2 -> 3).
    """
    return ((_sign_bit(y) << 3) | rne_to_grid(y, E2M1_GRID)).astype(np.uint8)


def e4m3_rne(y):
    """float -> E4M3FN code with round-to-nearest-even and saturation at 448."""
    return ((_sign_bit(y) << 7) | rne_to_grid(y, E4M3_GRID)).astype(np.uint8)


def sr_to_grid(y, u16, grid):
    """Stochastic rounding of |y| onto ``grid`` with a 16-bit uniform ``u16``.

    Reading of "Inkling 2 Small uses four-bit training ..." (ai-primer),
    section "Stochastic rounding across transposes": a value between two
    neighbouring grid values lo < hi rounds up with probability equal to its
    distance from lo as a fraction of the gap, which keeps its expectation.
    The pages fix the principle, not the random-bit rule; the rule taken here:

        D = (a - lo) / (hi - lo)        exact (the gaps are powers of two)
        P = floor(D * 2^16)
        round up  iff  u16 + P >= 2^16

    so the up-probability over all 2^16 values of u16 is exactly P / 2^16 and
    grid values (D = 0) never move. |y| must not exceed the grid maximum;
    |y| equal to it stays there. Returns magnitude indices.
    """
    a = np.abs(np.asarray(y, dtype=np.float64))
    if np.any(a > grid[-1]):
        raise ValueError("stochastic rounding input above the grid maximum")
    n = grid.shape[0]
    lo = np.searchsorted(grid, a, side="right") - 1
    lo = np.clip(lo, 0, n - 1)
    at_max = lo == n - 1
    hi = np.minimum(lo + 1, n - 1)
    gap = np.where(at_max, 1.0, grid[hi] - grid[lo])
    d = (a - grid[lo]) / gap
    p = np.floor(d * 65536.0).astype(np.int64)
    up = (np.asarray(u16).astype(np.int64) + p) >= 65536
    return np.where(at_max, lo, lo + up.astype(np.int64))


def e4m3_sr(y, u16):
    """float (|y| <= 448) -> E4M3FN code by stochastic rounding; keeps sign."""
    return ((_sign_bit(y) << 7) | sr_to_grid(y, u16, E4M3_GRID)).astype(np.uint8)


def e2m1_sr(y, u16):
    """float (|y| <= 6) -> E2M1 code by stochastic rounding; keeps sign."""
    return ((_sign_bit(y) << 3) | sr_to_grid(y, u16, E2M1_GRID)).astype(np.uint8)


# ---------------------------------------------------------------- E8M0 scale

def e8m0_ceil_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
    amax == 0 gives -127.

    Reading: the pages ask that re-quantization preserve forward values in
    expectation ("Stochastic rounding across transposes"). A block exponent
    that lets the block maximum land above 448 would force saturation (a
    biased result), so the exponent is the smallest one that keeps every
    element of the block inside the E4M3 range.
    """
    a = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(a)                 # a = f * 2^x, f in [0.5, 1)
    m = 2.0 * f                        # a = m * 2^(x-1), m in [1, 2)
    big_e = x - 1
    e = np.where(m <= 1.75, big_e - 8, big_e - 7)
    e = np.where(a == 0.0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


# ---------------------------------------------------------------- bfloat16

def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits_rne(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite x)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# ---------------------------------------------------------------- storage

def nvfp4_bits_per_value():
    """4-bit element plus an 8-bit scale shared by 16 elements."""
    return 4.0 + 8.0 / 16.0


def mxfp8_bits_per_value():
    """8-bit element plus an 8-bit scale shared by 32 elements."""
    return 8.0 + 8.0 / 32.0
