"""Pins of the oracle's MXFP8 quantizers: backward re-quantization with
stochastic rounding and round-to-nearest quantization of dY (CPU only).

Page facts checked ("Inkling 2 Small uses four-bit training ...", section
"Stochastic rounding across transposes"): re-quantization keeps the forward
values in expectation (the point of the recipe), and quantizing the two
orientations independently gives represented values that differ from the
forward ones. Section "Block scales and per-token activations": 8.25 bits per
value. Other tests are closed forms, brute force and an independent library
rounding (torch's float8_e4m3fn conversion).
"""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
from oracle import philox
from workloads import gen


def _saved(seed, rows, cols, per_group=None):
    x = gen.normal(seed, 0, (rows, cols))
    gen.with_outliers(x, seed, 6, frac=0.002)
    return Q.quantize(x, rows_per_group=per_group)


def test_rne_matches_torch_and_scale_rule():
    t = gen.normal(11, 0, (64, 256)) * np.float32(0.37)
    t[3] = 0.0
    t[5, :32] = np.float32(1e-30)
    codes, e8 = MX.quantize_rne(t)
    e = e8.astype(np.int64) - 127
    amax = np.abs(t).reshape(64, 8, 32).max(2).astype(np.float64)
    assert np.all(amax <= 448.0 * np.exp2(e))
    nz = amax > 0
    assert np.all(amax[nz] > 448.0 * np.exp2(e[nz] - 1))
    y = (t.reshape(64, 8, 32) * np.ldexp(np.float32(1), -e)[:, :, None].astype(np.float32)).astype(np.float32)
    ref = torch.from_numpy(y.reshape(64, 256)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # per-block max |y| lands in (224, 448]
    ym = np.abs(y).max(2)
    assert np.all((ym[nz] > 224) & (ym[nz] <= 448))
    assert codes.nbytes * 8 + e8.nbytes * 8 == 8.25 * t.size


def test_grouped_transpose_layout_bruteforce():
    rows, cols = 70, 64
    v = gen.normal(12, 0, (rows, cols))
    offsets = np.array([0, 5, 5, 40, 70])
    poff = MX.padded_offsets_from_offsets(offsets)
    assert list(poff) == [0, 32, 32, 96, 128]
    P = 128
    out = MX.transpose_grouped(v, offsets, poff, P)
    for k in range(cols):
        for p in range(P):
            want = 0.0
            for g in range(4):
                if poff[g] <= p < poff[g] + (offsets[g + 1] - offsets[g]):
                    want = v[offsets[g] + p - poff[g], k]
            assert out[k, p] == want


def test_requant_bracket_and_draw_mapping():
    codes, scales, outer = _saved(13, 96, 64)
    offsets = np.array([0, 33, 96])
    poff = MX.padded_offsets_from_offsets(offsets)
    P = int(poff[-1])
    seed, tag = 0x5EED0004, 0
    q8, e8 = MX.requant_sr(codes, scales, outer, offsets, poff, P, seed, tag)
    v = MX.transpose_grouped(Q.dequantize(codes, scales, outer), offsets, poff, P)
    e = e8.astype(np.int64) - 127
    y = (v.reshape(64, P // 32, 32) * np.ldexp(np.float32(1), -e)[:, :, None].astype(np.float32)
         ).astype(np.float32).reshape(64, P)
    got = F.e4m3_decode(q8)
    lo_i = np.searchsorted(F.E4M3_GRID, np.abs(y), side="right") - 1
    lo = F.E4M3_GRID[lo_i] * np.sign(y)
    hi = F.E4M3_GRID[np.minimum(lo_i + 1, 126)] * np.sign(y)
    assert np.all((got == lo) | (got == hi))
    # element (k, p) uses the draw at linear index k*P + p of the output
    r = np.random.default_rng(0)
    for _ in range(200):
        k, p = int(r.integers(0, 64)), int(r.integers(0, P))
        u = philox.uniform16(seed, tag, np.array([k * P + p]))[0]
        a = abs(float(y[k, p]))
        i = int(lo_i[k, p])
        if i == 126:
            continue
        D = (a - F.E4M3_GRID[i]) / (F.E4M3_GRID[i + 1] - F.E4M3_GRID[i])
        up = u + np.floor(D * 65536) >= 65536
        assert abs(got[k, p]) == F.E4M3_GRID[i + int(up)]
    # padding columns are zero, and the result is deterministic
    assert np.all(q8[:, 33:64] == 0)
    q8b, e8b = MX.requant_sr(codes, scales, outer, offsets, poff, P, seed, tag)
    assert np.array_equal(q8, q8b) and np.array_equal(e8, e8b)


def test_requant_on_grid_values_are_exact():
    """Saved values that already lie on the scaled E4M3 grid do not move for
    any seed: e2m1 * S with S in {1, 1.5, 2, 3} times a power-of-two outer
    scale has at most 4 significant bits, and the narrow ranges keep every
    value of a 32-block in the normal E4M3 range after block scaling."""
    r = np.random.default_rng(14)
    rows, cols = 64, 64
    c = r.integers(0, 16, (rows, cols)).astype(np.uint8)
    c[:, ::16] = 7                                              # top code in every block
    S_codes = r.choice([0x38, 0x3C, 0x40, 0x44], size=(rows, cols // 16)).astype(np.uint8)
    outer = np.ldexp(np.float32(1), r.integers(-8, -5, rows).astype(np.int32)).astype(np.float32)
    packed = Q.pack_codes(c)
    v = Q.dequantize(packed, S_codes, outer)
    offsets = np.array([0, rows])
    poff = MX.padded_offsets_from_offsets(offsets)
    for seed in (1, 2, 3):
        q8, e8 = MX.requant_sr(packed, S_codes, outer, offsets, poff, 64, seed, 0)
        assert np.array_equal(MX.dequantize(q8, e8), v.T.astype(np.float64))


def test_requant_unbiased_over_seeds():
    """Mean over 4096 seeds of the SR output converges to the dequantized
    forward value (expectation preserved, the reason for the recipe)."""
    codes, scales, outer = _saved(15, 32, 64)
    offsets = np.array([0, 32])
    poff = MX.padded_offsets_from_offsets(offsets)
    v = MX.transpose_grouped(Q.dequantize(codes, scales, outer), offsets, poff, 32).astype(np.float64)
    n = 4096
    acc = np.zeros_like(v)
    acc2 = np.zeros_like(v)
    for seed in range(n):
        q8, e8 = MX.requant_sr(codes, scales, outer, offsets, poff, 32, seed, 0)
        d = MX.dequantize(q8, e8)
        acc += d
        acc2 += d * d
    mean = acc / n
    var = np.maximum(acc2 / n - mean ** 2, 0)
    # per element within 5 standard errors, plus the bias of the 16-bit draw
    # resolution (at most 2^-16 of the largest E4M3 gap, 32 * 2^e)
    e = MX.block_exponents(v.astype(np.float32))
    gap_bound = np.repeat(np.exp2(e + 5).astype(np.float64), 32, axis=1)
    tol = 5 * np.sqrt(var / n) + gap_bound * 2.0 ** -16 + 1e-30
    assert np.all(np.abs(mean - v) <= tol)
    # the same seeds with round-to-nearest are biased on such data; SR is not
    assert np.abs((mean - v).mean()) < 1e-3 * np.abs(v).mean()


def _sr_sigma(y, e):
    """Analytic standard deviation of the mean SR error over the elements."""
    a = np.abs(y.astype(np.float64))
    lo_i = np.searchsorted(F.E4M3_GRID, a, side="right") - 1
    at_max = lo_i >= 126
    hi = F.E4M3_GRID[np.minimum(lo_i + 1, 126)]
    gap = np.where(at_max, 1.0, hi - F.E4M3_GRID[lo_i])
    D = (a - F.E4M3_GRID[lo_i]) / gap
    scale = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    var = np.where(at_max, 0.0, D * (1 - D)) * (gap * scale) ** 2
    return np.sqrt(var.sum()) / a.size


@pytest.mark.slow
def test_bias_check_1e7_elements():
    """Mean of SR outputs minus mean of inputs over 10^7 elements, against
    the analytic standard deviation; and an off-grid input where
    round-to-nearest is biased by -1/32 of the value and SR is not."""
    rows, cols = 5120, 2048                    # 1.05e7 elements
    codes, scales, outer = _saved(16, rows, cols)
    offsets = np.array([0, rows])
    poff = MX.padded_offsets_from_offsets(offsets)
    q8, e8 = MX.requant_sr(codes, scales, outer, offsets, poff, rows, 0x5EED0004, 0)
    v = MX.transpose_grouped(Q.dequantize(codes, scales, outer), offsets, poff, rows)
    d = MX.dequantize(q8, e8)
    e = e8.astype(np.int64) - 127
    y = (v.reshape(cols, rows // 32, 32) * np.ldexp(np.float32(1), -e)[:, :, None].astype(np.float32)
         ).reshape(cols, rows)
    sigma = _sr_sigma(y, e)
    bias = d.mean() - v.astype(np.float64).mean()
    assert abs(bias) <= 4 * sigma
    # off-grid constant 1.03125 * 2^j: RN rounds every element down by 1/32
    j = np.random.default_rng(17).integers(-10, 10, (64, 1))
    t = np.broadcast_to(np.ldexp(np.float32(1.03125), j.astype(np.int32)), (64, 4096)).astype(np.float32)
    rn = MX.dequantize(*MX.quantize_rne(t))
    sr = MX.dequantize(*MX.quantize_sr(t, 0x5EED0004, 2))
    rel_rn = (rn - t).mean(axis=1) / np.ldexp(1.0, j[:, 0])
    rel_sr = (sr - t).mean(axis=1) / np.ldexp(1.0, j[:, 0])
    assert np.allclose(rel_rn, -0.03125)
    # SR: D = 1/4 per element, per-row sd of the mean = 32*sqrt(3/16)/256/sqrt(4096)
    assert np.all(np.abs(rel_sr) <= 5 * 32 * np.sqrt(3 / 16) / 256 / 64)


def test_independent_orientations_differ_requant_does_not():
    """The failure mode the recipe fixes: quantizing W and W^T separately to
    NVFP4 gives represented values that differ from the forward's, while the
    SR re-quantization of the forward values is centred on them."""
    N, K = 64, 128
    w = gen.to_bf16_bits(gen.normal(18, 1, (N, K), std=0.02))
    fwd = Q.dequantize(*Q.quantize(w, rows_per_group=N), rows_per_group=N)            # [N, K]
    wt = np.ascontiguousarray(F.bf16_bits_to_f32(w).T)
    bwd_indep = Q.dequantize(*Q.quantize(wt, rows_per_group=K), rows_per_group=K).T   # [N, K]
    assert np.mean(bwd_indep != fwd) > 0.2
    codes, scales, outer = Q.quantize(w, rows_per_group=N)
    offsets = np.array([0, N])
    poff = MX.padded_offsets_from_offsets(offsets)
    n = 512
    acc = np.zeros((K, N))
    for seed in range(n):
        q8, e8 = MX.requant_sr(codes, scales, outer, offsets, poff, N, seed, 1, rows_per_group=N)
        acc += MX.dequantize(q8, e8)
    mean = acc / n
    err_sr = np.abs(mean - fwd.T).mean()
    err_indep = np.abs(bwd_indep - fwd).mean()
    assert err_sr < 0.1 * err_indep


def test_dy_orientations_agree_on_values():
    """Row-wise and grouped column-wise quantization of the same dY are two
    blockings of one tensor: both are within half an E4M3 step of it."""
    dy = gen.to_bf16_bits(gen.normal(19, 3, (100, 64), std=1e-3))
    x = F.bf16_bits_to_f32(dy).astype(np.float64)
    r8, re = MX.quantize_rowwise(dy)
    offsets = np.array([0, 31, 100])
    poff = MX.padded_offsets_from_offsets(offsets)
    c8, ce = MX.quantize_colwise_grouped(dy, offsets, poff, int(poff[-1]))
    rv = MX.dequantize(r8, re)
    cv = MX.transpose_grouped(MX.dequantize(c8, ce).T.astype(np.float32)[:, :], np.array([0, int(poff[-1])]),
                              np.array([0, int(poff[-1])]), int(poff[-1]))
    assert np.all(np.abs(rv - x) <= np.abs(x) * 2.0 ** -4 + 1e-30)
    back = np.concatenate([cv.T[0:31], cv.T[32:32 + 69]])
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + 1e-30)
    assert np.all(c8[:, 31:32] == 0)
