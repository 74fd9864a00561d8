"""Pins of the oracle's formats and rounding rules (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/pages_examples.json), closed forms, brute force, or
an independent library routine (torch's float8 conversions).
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import philox

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))


# ------------------------------------------------------------------ decoding

def test_e2m1_grid_is_the_fp4_grid():
    # the FP4 worked example has 4 and 6 as neighbouring grid values
    ex = GOLDEN["sr_worked_example"]
    grid = list(F.e2m1_decode(np.arange(8)))
    assert grid == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    i = grid.index(ex["lo"])
    assert grid[i + 1] == ex["hi"]
    # negative codes mirror the positive ones, code 8 is -0
    neg = F.e2m1_decode(np.arange(8, 16))
    assert np.all(neg == -np.array(grid))
    assert np.signbit(neg[0])


def test_e2m1_decode_matches_bitfields():
    # sign | 2-bit exponent (bias 1) | 1-bit mantissa, exponent 0 subnormal
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
        assert F.e2m1_decode(c) == (-v if s else v)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert F.e4m3_decode(0x7E) == 448.0 and F.e4m3_decode(0x08) == 2.0 ** -6
    assert F.e4m3_decode(0x01) == 2.0 ** -9 and F.e4m3_decode(0x38) == 1.0


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(F.e8m0_decode(codes), ref)
    assert np.isnan(F.e8m0_decode(255))


def test_bits_per_value_table():
    t = GOLDEN["bits_per_value"]
    assert F.nvfp4_bits_per_value() == t["NVFP4"]
    assert F.mxfp8_bits_per_value() == t["MXFP8"]
    assert round(t["BF16"] / F.nvfp4_bits_per_value(), 1) == GOLDEN["fewer_bits_than_bf16"]["ratio"]
    blk = GOLDEN["nvfp4_block"]
    assert F.nvfp4_bits_per_value() == 4 + blk["scale_bits"] / blk["values_per_scale"]


# ------------------------------------------------------------------ RNE

def _nearest_even_bruteforce(a, grid):
    """argmin |a - g| over the grid, ties to the even index, saturating."""
    d = np.abs(grid[None, :] - a[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.where(cand.sum(1) > 1, np.argmax(cand & (np.arange(grid.size) % 2 == 0), axis=1),
                   np.argmax(cand, axis=1))
    return np.where(a >= grid[-1], grid.size - 1, idx)


def test_rn_illustration_from_pages():
    ex = GOLDEN["rn_illustration"]
    grid = np.array(ex["grid"])
    i = F.rne_to_grid(np.array([ex["value"]]), grid)[0]
    assert grid[i] == ex["rounded"]
    assert abs(abs(ex["value"] - grid[i]) - ex["error"]) < 1e-12


def test_e2m1_rne_ties_and_bruteforce():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, want in ties.items():
        for sgn in (1, -1):
            c = F.e2m1_rne(np.float32(sgn * y))
            assert F.e2m1_decode(c) == sgn * want
    # every midpoint and its float32 neighbours, plus a dense sweep
    g = F.E2M1_GRID.astype(np.float32)
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10)),
                          np.linspace(0, 9, 20001, dtype=np.float32), g])
    got = F.rne_to_grid(pts, F.E2M1_GRID)
    assert np.array_equal(got, _nearest_even_bruteforce(pts.astype(np.float64), F.E2M1_GRID))
    assert F.e2m1_decode(F.e2m1_rne(np.float32(100.0))) == 6.0    # saturation
    assert F.e2m1_rne(np.float32(-0.0)) == 0x8                     # sign of zero kept


def test_e4m3_rne_matches_torch():
    g = F.E4M3_GRID.astype(np.float32)
    mids = ((g[:-1].astype(np.float64) + g[1:]) / 2).astype(np.float32)
    r = np.random.default_rng(0)
    pts = np.concatenate([
        g, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
        r.uniform(0, 448, 100000).astype(np.float32),
        np.exp2(r.uniform(-14, 8.8, 100000)).astype(np.float32),
    ])
    pts = pts[pts <= 448]
    pts = np.concatenate([pts, -pts])
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_rne(pts), ref)
    # saturation above 448 (torch would produce NaN past 464)
    assert F.e4m3_rne(np.float32(500.0)) == 0x7E
    assert F.e4m3_rne(np.float32(-1e30)) == 0xFE


# ------------------------------------------------------------------ SR

def test_sr_worked_example_exhaustive():
    ex = GOLDEN["sr_worked_example"]
    u = np.arange(65536)
    c = F.e2m1_sr(np.full(65536, ex["value"], np.float32), u)
    vals = F.e2m1_decode(c)
    assert set(np.unique(vals)) == {ex["lo"], ex["hi"]}
    assert np.sum(vals == ex["hi"]) == int(ex["p_hi"] * 65536)
    assert np.sum(vals == ex["lo"]) == int(ex["p_lo"] * 65536)
    assert vals.mean() == ex["expectation"]


def test_sr_worked_example_philox_1e6():
    ex = GOLDEN["sr_worked_example"]
    n = 10 ** 6
    u = philox.uniform16_range(0x5EED0001, 0, 0, n)
    vals = F.e2m1_decode(F.e2m1_sr(np.full(n, ex["value"], np.float32), u))
    k = int(np.sum(vals == ex["hi"]))
    sigma = np.sqrt(n * ex["p_hi"] * ex["p_lo"])
    assert abs(k - n * ex["p_hi"]) <= 5 * sigma
    assert abs(vals.mean() - ex["expectation"]) <= 5 * 2.0 * np.sqrt(ex["p_hi"] * ex["p_lo"] / n)


@pytest.mark.parametrize("grid_name", ["e2m1", "e4m3"])
def test_sr_bracket_identity_and_frequency(grid_name):
    grid = F.E2M1_GRID if grid_name == "e2m1" else F.E4M3_GRID
    enc = F.e2m1_sr if grid_name == "e2m1" else F.e4m3_sr
    dec = F.e2m1_decode if grid_name == "e2m1" else F.e4m3_decode
    # grid values never move, for any draw
    u = np.arange(0, 65536, 257)
    for gv in grid:
        out = dec(enc(np.full(u.size, gv, np.float32), u))
        assert np.all(out == gv)
    # exhaustive over u for points at known fractions of a gap
    r = np.random.default_rng(1)
    lo_idx = r.integers(0, grid.size - 1, 40)
    for i in lo_idx:
        lo, hi = grid[i], grid[i + 1]
        for frac in (1 / 65536, 0.125, 0.3, 0.5, 0.75, 1 - 1 / 65536):
            y = np.float32(lo + frac * (hi - lo))
            D = (np.float64(y) - lo) / (hi - lo)
            uu = np.arange(65536)
            out = dec(enc(np.full(65536, y, np.float32), uu))
            assert set(np.unique(out)) <= {lo, hi}
            assert np.sum(out == hi) == np.floor(D * 65536)
    with pytest.raises(ValueError):
        enc(np.float32(grid[-1] * 1.01), 0)


# ------------------------------------------------------------------ E8M0

def test_e8m0_ceil_is_smallest_exponent():
    r = np.random.default_rng(2)
    a = np.concatenate([
        np.exp2(r.uniform(-100, 100, 20000)),
        448.0 * np.exp2(np.arange(-100, 100)),                 # exact boundaries
        np.nextafter(448.0 * np.exp2(np.arange(-100, 100)), np.inf),
        [1.75, 1.75 * 2 ** 5, 1.8, 1.0, 2.0 ** -126, 3e38],
    ]).astype(np.float32).astype(np.float64)
    e = F.e8m0_ceil_exponent(a)
    assert np.all(a <= 448.0 * np.exp2(e.astype(np.float64)))
    unclamped = e > -127
    assert np.all(a[unclamped] > 448.0 * np.exp2(e[unclamped].astype(np.float64) - 1))
    assert F.e8m0_ceil_exponent(2.0 ** -126) == -127               # clamp
    assert F.e8m0_ceil_exponent(0.0) == -127
    assert F.e8m0_ceil_exponent(448.0) == 0 and F.e8m0_ceil_exponent(449.0) == 1


def test_bf16_round_trip_and_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -3.5, 0.0], np.float32)
    bits = F.f32_to_bf16_bits_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    r = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits_rne(r), ref)
    assert np.array_equal(F.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())
