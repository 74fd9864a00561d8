"""Pins of the oracle's permutation and grouped matmuls (CPU only).

Permutation: brute force with plain Python loops over experts and tokens.
Matmuls: exact rational arithmetic (fractions.Fraction) on small cases where
the float32 result must be exact; float32 vs float64 within the summation
error bound; brute-force index loops for the dgrad/wgrad layouts; and the
rank-1 outer-scale epilogue.
"""

from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
from oracle import permute as PM
from workloads import gen


# ------------------------------------------------------------------ permute

def _permute_bruteforce(topk, e0, n_local):
    T, k = topk.shape
    rows = []
    counts = []
    for e in range(e0, e0 + n_local):
        c = 0
        for t in range(T):
            for j in range(k):
                if topk[t, j] == e:
                    rows.append((t, j))
                    c += 1
        counts.append(c)
    offsets = [0]
    padded = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
        padded.append(padded[-1] + (c + 31) // 32 * 32)
    return offsets, padded, [r[0] for r in rows], [r[1] for r in rows]


def test_permute_bruteforce_uniform_and_zipf():
    cases = [
        (gen.route_uniform(21, 37, 8, 2), 0, 8),
        (gen.route_uniform(22, 50, 64, 8), 16, 8),       # only some experts local
        (gen.route_zipf(23, 64, k=8, n_experts=64), 8, 8),
        (np.zeros((5, 1), np.int32), 0, 1),
        (np.full((6, 2), 3, np.int32)[:0], 0, 4),       # no tokens
    ]
    for topk, e0, nl in cases:
        off, pad, rt, rs = PM.permute(topk, e0, nl)
        bo, bp, brt, brs = _permute_bruteforce(topk, e0, nl)
        assert list(off) == bo and list(pad) == bp
        assert list(rt) == brt and list(rs) == brs
        assert all(p % 32 == 0 for p in pad)


def test_gather_rows():
    x = gen.normal(24, 0, (10, 32))
    codes, scales, outer = Q.quantize(x)
    topk = gen.route_uniform(24, 10, 4, 2)
    off, pad, rt, rs = PM.permute(topk, 0, 4)
    c2, s2, o2 = PM.gather_rows(rt, codes, scales, outer)
    for r in range(len(rt)):
        assert np.array_equal(c2[r], codes[rt[r]]) and o2[r] == outer[rt[r]]
        assert topk[rt[r], rs[r]] == np.searchsorted(off, r, side="right") - 1


# ------------------------------------------------------------------ matmuls

def _exact_forward(A, B, sx, sw, offsets):
    """Exact rational Y for small cases."""
    M, K = A.shape
    G, N, _ = B.shape
    Y = [[None] * N for _ in range(M)]
    for g in range(G):
        for r in range(offsets[g], offsets[g + 1]):
            for n in range(N):
                acc = sum(Fraction(float(A[r, k])) * Fraction(float(B[g, n, k])) for k in range(K))
                Y[r][n] = acc * Fraction(float(sx[r])) * Fraction(float(sw[g]))
    return Y


def test_forward_exact_case():
    """Power-of-two outer scales and a short contraction: every partial sum
    is exact in float32, so the float32 result must equal the exact value."""
    r = np.random.default_rng(25)
    M, K, N, G = 12, 32, 8, 2
    x = r.standard_normal((M, K)).astype(np.float32)
    w = r.standard_normal((G * N, K)).astype(np.float32)
    ac, asc, _ = Q.quantize(x)
    bc, bsc, _ = Q.quantize(w, rows_per_group=N)
    # exact-friendly scales: restrict block scales to a narrow range
    asc[:] = np.where(asc > 0, 0x38 + (asc & 3), 0).astype(np.uint8)
    bsc[:] = np.where(bsc > 0, 0x38 + (bsc & 3), 0).astype(np.uint8)
    sx = np.ldexp(np.float32(1), r.integers(-10, 10, M).astype(np.int32)).astype(np.float32)
    sw = np.ldexp(np.float32(1), r.integers(-10, 10, G).astype(np.int32)).astype(np.float32)
    offsets = np.array([0, 5, 12])
    Y = GM.fwd_grouped(ac, asc, sx, bc.reshape(G, N, K // 2), bsc.reshape(G, N, K // 16), sw, offsets, N)
    A = Q.dequantize(ac, asc, None, apply_outer=False)
    B = Q.dequantize(bc, bsc, None, apply_outer=False).reshape(G, N, K)
    ex = _exact_forward(A, B, sx, sw, offsets)
    for i in range(M):
        for n in range(N):
            assert Fraction(float(Y[i, n])) == ex[i][n]


def test_forward_fp32_close_to_fp64_and_rank1_epilogue():
    case = gen.moe_case(26, T=96, K=256, N=64, E=4, k=2)
    xc, xs, xo = Q.quantize(case["x"])
    wc, ws, wo = Q.quantize(case["w"], rows_per_group=case["N"])
    off, pad, rt, rs = PM.permute(case["topk"], 0, 4)
    ac, asc, ao = PM.gather_rows(rt, xc, xs, xo)
    G, N, K = 4, 64, 256
    bc, bsc = wc.reshape(G, N, K // 2), ws.reshape(G, N, K // 16)
    y32 = GM.fwd_grouped(ac, asc, ao, bc, bsc, wo, off, N)
    y64 = GM.fwd_grouped(ac, asc, ao, bc, bsc, wo, off, N, accum="fp64")
    # |fl32(sum) - sum| <= K * 2^-24 * sum|terms| (plus two epilogue roundings)
    A = Q.dequantize(ac, asc, None, apply_outer=False).astype(np.float64)
    B = Q.dequantize(wc, ws, None, apply_outer=False).reshape(G, N, K).astype(np.float64)
    for g in range(G):
        a, b = off[g], off[g + 1]
        absum = np.abs(A[a:b]) @ np.abs(B[g]).T * ao[a:b, None] * wo[g]
        assert np.all(np.abs(y32[a:b] - y64[a:b]) <= (K + 3) * 2.0 ** -24 * absum + 1e-30)
    # doubling one token's outer scale doubles its row exactly
    ao2 = ao.copy()
    ao2[3] *= 2
    y2 = GM.fwd_grouped(ac, asc, ao2, bc, bsc, wo, off, N)
    assert np.array_equal(y2[3], 2 * y32[3])
    assert np.array_equal(np.delete(y2, 3, 0), np.delete(y32, 3, 0))


def test_dgrad_wgrad_bruteforce_layouts():
    r = np.random.default_rng(27)
    G, N, K = 2, 64, 32
    offsets = np.array([0, 7, 40])
    poff = MX.padded_offsets_from_offsets(offsets)
    M, P = 40, int(poff[-1])
    dy = r.standard_normal((M, N)).astype(np.float32)
    wT = r.standard_normal((K, G * N)).astype(np.float32)
    xT = r.standard_normal((K, P)).astype(np.float32)
    dy8, dye = MX.quantize_rne(dy)
    w8, we = MX.quantize_rne(wT)
    dyT8, dyTe = MX.quantize_colwise_grouped(dy, offsets, poff, P)
    x8, xe = MX.quantize_rne(xT)
    dX = GM.dgrad_grouped(dy8, dye, w8, we, offsets, N, accum="fp64")
    dW = GM.wgrad_grouped(dyT8, dyTe, x8, xe, poff, accum="fp64")
    DY, W, DYT, X = (MX.dequantize(a, b) for a, b in ((dy8, dye), (w8, we), (dyT8, dyTe), (x8, xe)))
    for g in range(G):
        for rr in range(offsets[g], offsets[g + 1]):
            for k in range(0, K, 7):
                s = sum(Fraction(DY[rr, n]) * Fraction(W[k, g * N + n]) for n in range(N))
                assert abs(float(s) - dX[rr, k]) <= 1e-12 * max(1.0, abs(float(s)))
        for n in range(0, N, 9):
            for k in range(0, K, 5):
                s = sum(Fraction(DYT[n, p]) * Fraction(X[k, p]) for p in range(poff[g], poff[g + 1]))
                assert abs(float(s) - dW[g, n, k]) <= 1e-12 * max(1.0, abs(float(s)))
    # the grouped transpose of dY holds dY's rows of group g in g's columns
    assert np.array_equal(DYT[:, poff[1]:poff[1] + 33], MX.dequantize(*MX.quantize_rne(
        np.ascontiguousarray(np.pad(dy[7:40].T, ((0, 0), (0, 31))))))[:, :33])
    assert F.E4M3_MAX == 448.0


def test_forward_mxfp8_bruteforce_and_fp32_bound():
    """The all-MXFP8 forward: exact sums by brute force over k on sampled
    outputs (every dequantized product is exact), and float32 accumulation
    within the summation error bound of the exact sum."""
    r = np.random.default_rng(28)
    G, N, K = 3, 32, 96
    offsets = np.array([0, 5, 5, 23])
    M = int(offsets[-1])
    x = (r.standard_normal((M, K)) * np.exp2(r.integers(-6, 6, (M, 1)))).astype(np.float32)
    w = (r.standard_normal((G * N, K)) * 0.05).astype(np.float32)
    x8, xe = MX.quantize_rne(x)
    w8, we = MX.quantize_rne(w)
    y64 = GM.fwd_grouped_mxfp8(x8, xe, w8.reshape(G, N, K), we.reshape(G, N, K // 32), offsets, N,
                               accum="fp64")
    y32 = GM.fwd_grouped_mxfp8(x8, xe, w8, we, offsets, N)
    X, W = MX.dequantize(x8, xe), MX.dequantize(w8, we).reshape(G, N, K)
    for g in range(G):
        for rr in range(offsets[g], offsets[g + 1]):
            for n in range(0, N, 5):
                s = sum(Fraction(float(X[rr, k])) * Fraction(float(W[g, n, k])) for k in range(K))
                assert abs(float(s) - y64[rr, n]) <= 1e-12 * max(1.0, abs(float(s)))
                bound = K * 2.0 ** -24 * float(sum(abs(Fraction(float(X[rr, k])) * Fraction(float(W[g, n, k])))
                                                   for k in range(K)))
                assert abs(float(y32[rr, n]) - float(s)) <= bound + 1e-30
    # rows of an empty group: none; rows past offsets[-1]: none
    assert y32.shape == (M, N)
