"""Pins of the oracle's NVFP4 quantizer (CPU only).

What the pages fix ("Inkling 2 Small uses four-bit training ...", section
"Block scales and per-token activations"): 16 values share one E4M3 scale,
4.5 bits per value, an FP32 outer scale per token (independent of other
tokens) or per expert. The tests check those facts, plus properties that hold
for any correct implementation of the stated reading: the largest block of a
nonzero row gets the top E4M3 scale and its largest element the top E2M1 code,
round-to-nearest error bounds, exact round trips of representable values, and
the nibble/row/block layout.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as Q
from workloads import gen


def _rows(seed, rows, cols, outliers=True):
    x = gen.normal(seed, 0, (rows, cols))
    if outliers:
        gen.with_outliers(x, seed, 6, frac=0.01)
    return x


def test_storage_is_4p5_bits_per_value():
    x = _rows(1, 8, 256)
    codes, scales, outer = Q.quantize(x)
    n = x.size
    assert codes.nbytes * 8 + scales.nbytes * 8 == 4.5 * n
    assert scales.shape == (8, 256 // 16) and codes.shape == (8, 128)


def test_top_scale_and_top_code_in_every_nonzero_row():
    x = _rows(2, 64, 512)
    codes, scales, outer = Q.quantize(x)
    c = Q.unpack_codes(codes)
    assert np.all(np.any(scales == 0x7E, axis=1))
    assert np.all(np.any((c & 7) == 7, axis=1))
    assert np.all(scales != 0x7F) and np.all(scales < 0x80)      # no NaN, never negative
    assert np.array_equal(outer, (np.abs(x).max(1) / np.float32(2688)).astype(np.float32))


def test_zero_rows_and_signed_zeros():
    x = _rows(3, 4, 64)
    x[1] = 0.0
    x[2] = -0.0
    codes, scales, outer = Q.quantize(x)
    c = Q.unpack_codes(codes)
    assert outer[1] == 0 and outer[2] == 0
    assert np.all(scales[1:3] == 0)
    assert np.all(c[1] == 0) and np.all(c[2] == 8)
    v = Q.dequantize(codes, scales, outer)
    assert np.all(v[1:3] == 0) and np.all(np.signbit(v[2]))


def test_round_to_nearest_error_bound():
    x = _rows(4, 128, 1024)
    codes, scales, outer = Q.quantize(x)
    c = Q.unpack_codes(codes)
    S = F.e4m3_decode(scales).astype(np.float64)
    unit = np.repeat(S, 16, axis=1) * outer[:, None].astype(np.float64)      # S * s per element
    v = Q.dequantize(codes, scales, outer).astype(np.float64)
    mag = c & 7
    # gap above each code magnitude (the grid spacing around the value)
    gaps = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])[mag]
    y = np.abs(x.astype(np.float64)) / unit
    unsat = y <= 6.0
    err = np.abs(x.astype(np.float64) - v)
    bound = 0.5 * gaps * unit * (1 + 1e-5) + 1e-30
    assert np.all(err[unsat] <= bound[unsat])
    # saturated elements sit at 6 and exceed it by less than the scale's own rounding (1/16)
    assert np.all(mag[~unsat] == 7)
    assert np.all(y[~unsat] <= 6.0 * (1 + 1 / 16) * (1 + 1e-5))


def test_bruteforce_every_code_and_scale_round_trips():
    """One-block rows whose values are exactly e2m1(c) * S for all 16 codes,
    for every positive finite E4M3 scale S: re-quantizing gives back the same
    codes and the top scale 0x7E (the outer scale absorbs S)."""
    base = np.arange(16)
    rows = []
    perms = [base, base[::-1], np.roll(base, 5)]
    for s_code in range(1, 0x7F):
        S = F.e4m3_decode(s_code)
        for p in perms:
            rows.append((p, F.e2m1_decode(p) * S))
    codes_in = np.array([r[0] for r in rows], np.uint8)
    x = np.array([r[1] for r in rows], np.float32)
    codes, scales, outer = Q.quantize(x)
    assert np.all(scales[:, 0] == 0x7E)
    got = Q.unpack_codes(codes)
    # +0 and -0 both encode zero; compare values and signs of nonzeros
    assert np.array_equal(F.e2m1_decode(got), F.e2m1_decode(codes_in))


def test_tokens_are_independent():
    x = _rows(5, 32, 256)
    codes, scales, outer = Q.quantize(x)
    for i in (0, 7, 31):
        c1, s1, o1 = Q.quantize(x[i:i + 1])
        assert np.array_equal(c1[0], codes[i]) and np.array_equal(s1[0], scales[i]) and o1[0] == outer[i]


def test_per_expert_outer_scale():
    E, N, K = 3, 32, 128
    w = gen.normal(6, 1, (E * N, K), std=0.02)
    codes, scales, outer = Q.quantize(w, rows_per_group=N)
    assert outer.shape == (E,)
    for e in range(E):
        blk = w[e * N:(e + 1) * N]
        assert outer[e] == np.float32(np.abs(blk).max() / np.float32(2688))
        assert np.any(scales[e * N:(e + 1) * N] == 0x7E)
    # one row per group is the per-token quantizer
    c1, s1, o1 = Q.quantize(w, rows_per_group=1)
    c2, s2, o2 = Q.quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(o1, o2)
    # a group's quantization does not depend on other groups
    c3, s3, o3 = Q.quantize(w[N:2 * N], rows_per_group=N)
    assert np.array_equal(c3, codes[N:2 * N]) and o3[0] == outer[1]


def test_layout_nibbles_blocks_rows():
    x = np.zeros((2, 32), np.float32)
    x[0, 1] = 6.0          # element 1: high nibble of byte 0
    x[0, 0] = 1.0          # element 0: low nibble of byte 0
    x[1, 17] = -3.0        # row 1, block 1, element 17: high nibble of byte 8
    codes, scales, outer = Q.quantize(x)
    assert codes[0, 0] == (0x7 << 4) | 0x2
    assert np.all(codes[0, 1:] == 0)
    assert codes[1, 8] == (0xF << 4)               # -6 (the row max) in the high nibble
    assert scales[0, 0] == 0x7E and scales[0, 1] == 0
    assert scales[1, 0] == 0 and scales[1, 1] == 0x7E
    assert outer[0] == np.float32(6.0) / np.float32(2688) and outer[1] == np.float32(3.0) / np.float32(2688)


def test_bf16_input_equals_its_float32_value():
    x = gen.to_bf16_bits(_rows(7, 16, 128))
    a = Q.quantize(x)
    b = Q.quantize(F.bf16_bits_to_f32(x))
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 24), np.float32))
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((5, 16), np.float32), rows_per_group=2)
