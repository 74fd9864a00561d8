"""Pins of the oracle's NVFP4 backward (CPU only).

* E4M3 rounding up: brute force over the whole E4M3 grid.
* Row-wise and grouped-transposed NVFP4 with stochastic rounding: inputs built
  to be exactly representable come back exactly for every seed (this fixes the
  rounded-up block scale, the outer scale per row / per group, the transpose
  and the group placement: any other choice leaves values off the grid, where
  stochastic rounding moves them); the mean over many seeds equals the input
  within the sampling error (unbiased); padding is zero.
* Per-expert transposed weights: exact round trip on representable weights.
* dgrad / wgrad: plain index loops over the dequantized operands.
* The backward's weight gradient is unbiased over seeds; the same operands
  rounded to nearest are not.
"""

import numpy as np

from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import nvfp4_bwd as NB
from workloads import gen

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e4m3_ceil_bruteforce():
    grid = F.E4M3_GRID.astype(np.float64)
    for c in range(127):
        assert NB.e4m3_ceil(grid[c]) == c
        if c < 126:
            assert NB.e4m3_ceil(np.nextafter(grid[c], np.inf)) == c + 1
        if c > 0:
            assert NB.e4m3_ceil(np.nextafter(grid[c], 0.0)) == c
    assert NB.e4m3_ceil(0.0) == 0 and NB.e4m3_ceil(1e9) == 126
    t = np.random.default_rng(3).random(2000) * 500
    for v in t:
        expect = min([c for c in range(127) if grid[c] >= v] or [126])
        assert NB.e4m3_ceil(v) == expect


def test_e2m1_sr_saturates_above_six():
    assert NB.e2m1_sr_sat(np.float32(6.0000005), np.uint32(65535)) == 7
    assert NB.e2m1_sr_sat(np.float32(-6.5), np.uint32(0)) == 15
    # the pages' worked example: 4.5 between 4 and 6 rounds up iff u >= 3/4 of 2^16
    assert NB.e2m1_sr_sat(4.5, np.uint32(49151)) == 6
    assert NB.e2m1_sr_sat(4.5, np.uint32(49152)) == 7


def _representable_rows(R, nblocks, seed):
    """Rows whose NVFP4 form is exact: block b holds E2M1 values times 2^j_b,
    and the first block reaches 6 * 448 = 2688 so that s = 1 exactly."""
    rng = np.random.default_rng(seed)
    x = np.zeros((R, 16 * nblocks), np.float32)
    for r in range(R):
        for b in range(nblocks):
            v = rng.choice(E2M1, 16) * rng.choice([-1.0, 1.0], 16)
            v[rng.integers(16)] = 6.0
            x[r, 16 * b:16 * b + 16] = v * (448.0 if b == 0 else 2.0 ** int(rng.integers(-6, 7)))
    return x


def test_rows_exact_when_representable():
    x = _representable_rows(6, 5, 1)
    for seed in (1, 2, 3):
        c, s, o = NB.quantize_sr_rows(x, seed)
        assert np.all(o == 1.0)
        assert np.array_equal(Q.dequantize(c, s, o), x)


def test_rows_unbiased():
    x = gen.normal(11, 0, (4, 64))
    gen.with_outliers(x, 11, 6, frac=0.05, factor=20.0)
    n = 3000
    acc = np.zeros(x.shape)
    acc2 = np.zeros(x.shape)
    for seed in range(n):
        v = Q.dequantize(*NB.quantize_sr_rows(x, seed)).astype(np.float64)
        acc += v
        acc2 += v * v
    mean = acc / n
    sd = np.sqrt(np.maximum(acc2 / n - mean ** 2, 0))
    # Each element sits between two grid neighbours a gap g apart and rounds up
    # with probability p = its fractional position; the mean of n draws is within
    # 5 g sqrt(p (1 - p) / n) of it, plus g * 6 / n for rare up-moves and 2^-16 g
    # for the 16-bit draw (p is floored to a multiple of 2^-16). Scales do not
    # depend on the seed.
    _, sc, o = NB.quantize_sr_rows(x, 0)
    unit = np.repeat(F.e4m3_decode(sc), 16, axis=1) * o[:, None]        # S s
    a = np.abs(x) / unit
    g = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    pfrac = a / g - np.floor(a / g)
    gap = g * unit
    bound = 5 * gap * np.sqrt(pfrac * (1 - pfrac) / n) + 6 * gap / n + gap * 2.0 ** -16
    assert np.all(np.abs(mean - x) <= bound)
    # round to nearest is biased on the same values
    rne = Q.dequantize(*Q.quantize(x)).astype(np.float64)
    assert np.abs(rne - x).max() > 10 * np.abs(mean - x).max()


def test_grouped_transpose_exact_and_padded():
    # rows of 3 groups; transposed, each output row's 16-blocks must hold E2M1 values
    # times one power of two, and each group's maximum 2688 (so its outer scale is 1)
    lens = [40, 0, 23, 64]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    poff = NB.padded_offsets(off)
    assert np.array_equal(poff, [0, 128, 128, 256, 384])
    cols = 48
    rng = np.random.default_rng(4)
    v = np.zeros((off[-1], cols), np.float32)
    for g in range(4):
        a, b = int(off[g]), int(off[g + 1])
        for c in range(cols):
            for p0 in range(a, b, 16):
                p1 = min(p0 + 16, b)
                vals = rng.choice(E2M1, p1 - p0) * rng.choice([-1.0, 1.0], p1 - p0)
                vals[rng.integers(p1 - p0)] = 6.0          # each block reaches 6 * its unit
                first = c == 0 and p0 == a                 # the group maximum 6 * 448
                v[p0:p1, c] = vals * (448.0 if first else 2.0 ** int(rng.integers(-4, 6)))
    P = int(poff[-1]) + 128
    for seed in (5, 6):
        codes, scales, outer = NB.quantize_sr_grouped_T(v, off, poff, P, seed, NB.TAG_X)
        assert np.array_equal(outer, [1.0, 0.0, 1.0, 1.0])
        back = Q.dequantize(codes, scales, np.ones(cols, np.float32))
        for g in range(4):
            a, b, p = int(off[g]), int(off[g + 1]), int(poff[g])
            assert np.array_equal(back[:, p:p + b - a], v[a:b].T)
            assert np.all(back[:, p + b - a:int(poff[g + 1])] == 0)
        assert np.all(codes[:, int(poff[-1]) // 2:] == 0)


def test_grouped_transpose_unbiased():
    v = gen.normal(12, 0, (50, 8))
    off = np.array([0, 20, 50], np.int64)
    poff = NB.padded_offsets(off)
    P = int(poff[-1])
    n = 800
    acc = np.zeros((8, P))
    for seed in range(n):
        c, s, o = NB.quantize_sr_grouped_T(v, off, poff, P, seed, NB.TAG_X)
        og = np.zeros(P, np.float32)
        for g in range(2):
            og[poff[g]:poff[g + 1]] = o[g]
        acc += Q.dequantize(c, s, None, apply_outer=False).astype(np.float64) * og
    mean = acc / n
    for g in range(2):
        a, b, p = int(off[g]), int(off[g + 1]), int(poff[g])
        ref = v[a:b].T.astype(np.float64)
        gap = 2.0 * np.abs(ref).max() / 6.0                   # largest possible gap
        assert np.all(np.abs(mean[:, p:p + b - a] - ref) <= 5 * gap / np.sqrt(n))


def test_weights_transposed_per_expert_exact():
    E, N, K = 3, 32, 48
    rng = np.random.default_rng(7)
    # exact in both orientations: 16x16 tiles of E2M1 values times one unit, the
    # tile's diagonal at 6 units (every block along n and along k reaches it);
    # expert e's first tile has unit 448 * 2^e, so its outer scale is 2^e
    w = np.zeros((E * N, K), np.float32)
    for e in range(E):
        for n0 in range(0, N, 16):
            for k0 in range(0, K, 16):
                t = rng.choice(E2M1, (16, 16)) * rng.choice([-1.0, 1.0], (16, 16))
                np.fill_diagonal(t, 6.0)
                unit = 448.0 if n0 == 0 and k0 == 0 else 2.0 ** int(rng.integers(-3, 4))
                w[e * N + n0:e * N + n0 + 16, k0:k0 + 16] = t * unit * 2.0 ** e
    wq = Q.quantize(w, rows_per_group=N)
    deq = Q.dequantize(*wq, rows_per_group=N).reshape(E, N, K)
    assert np.array_equal(deq, w.reshape(E, N, K))               # the forward form is exact
    c, s, o = NB.requant_weights_sr(*wq, E, seed=9)
    back = Q.dequantize(c, s, o, rows_per_group=K).reshape(E, K, N)
    assert np.array_equal(o, [2.0 ** e for e in range(E)])
    assert np.array_equal(back, deq.transpose(0, 2, 1))


def test_dgrad_wgrad_index_loops():
    rng = np.random.default_rng(8)
    M, N, K, E = 40, 32, 48, 3
    off = np.array([0, 13, 13, 40], np.int64)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    dyq = NB.quantize_sr_rows(dy, 1)
    w = rng.standard_normal((E * N, K)).astype(np.float32)
    wT = NB.requant_weights_sr(*Q.quantize(w, rows_per_group=N), E, seed=2)
    dx = NB.dgrad(dyq, wT, off, K, accum="fp64")
    A = Q.dequantize(dyq[0], dyq[1], None, apply_outer=False).astype(np.float64)
    Bw = Q.dequantize(wT[0], wT[1], None, apply_outer=False).astype(np.float64)   # [E*K, N]
    for r in range(M):
        g = int(np.searchsorted(off, r, side="right") - 1)
        for k in range(K):
            ref = sum(A[r, n] * Bw[g * K + k, n] for n in range(N))
            ref *= float(dyq[2][r]) * float(wT[2][g])
            assert abs(dx[r, k] - ref) <= 1e-9 * (1 + abs(ref))
    poff = NB.padded_offsets(off)
    P = int(poff[-1])
    x = rng.standard_normal((M, K)).astype(np.float32)
    dyT = NB.quantize_sr_grouped_T(dy, off, poff, P, 3, NB.TAG_DY_COL)
    xT = NB.quantize_sr_grouped_T(x, off, poff, P, 3, NB.TAG_X)
    dw = NB.wgrad(dyT, xT, poff, accum="fp64")
    Ad = Q.dequantize(dyT[0], dyT[1], None, apply_outer=False).astype(np.float64)
    Bd = Q.dequantize(xT[0], xT[1], None, apply_outer=False).astype(np.float64)
    for g in range(E):
        for n in range(0, N, 7):
            for k in range(0, K, 5):
                ref = sum(Ad[n, p] * Bd[k, p] for p in range(poff[g], poff[g + 1]))
                ref *= float(dyT[2][g]) * float(xT[2][g])
                assert abs(dw[g, n, k] - ref) <= 1e-9 * (1 + abs(ref))


def test_weight_gradient_unbiased_over_seeds():
    M, N, K = 64, 16, 16
    dy = gen.normal(13, 3, (M, N))
    x = gen.normal(13, 0, (M, K))
    off = np.array([0, M], np.int64)
    poff = NB.padded_offsets(off)
    exact = dy.astype(np.float64).T @ x.astype(np.float64)
    n = 400
    acc = np.zeros((N, K))
    for seed in range(n):
        dyT = NB.quantize_sr_grouped_T(dy, off, poff, int(poff[-1]), seed, NB.TAG_DY_COL)
        xT = NB.quantize_sr_grouped_T(x, off, poff, int(poff[-1]), seed, NB.TAG_X)
        acc += NB.wgrad(dyT, xT, poff, accum="fp64")[0]
    mean = acc / n
    one = NB.wgrad(NB.quantize_sr_grouped_T(dy, off, poff, int(poff[-1]), 0, NB.TAG_DY_COL),
                   NB.quantize_sr_grouped_T(x, off, poff, int(poff[-1]), 0, NB.TAG_X),
                   poff, accum="fp64")[0]
    spread = np.abs(one - exact).mean()
    # the mean over seeds converges to the exact product: error shrinks ~ 1/sqrt(n)
    assert np.abs(mean - exact).mean() < 4 * spread / np.sqrt(n)
