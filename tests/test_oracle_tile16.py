"""Pins of the oracle's 16x16-tile NVFP4 variant and the ablation against
1x16 blocks (CPU only).

The tile variant is the alternative the pages report rejecting ("Inkling 2
Small uses four-bit training ...", section "Stochastic rounding across
transposes"): transpose-invariant, but one large value pushes the rest of
its tile to zero. Pins: the representation of W^T is the transpose of that
of W (the property the variant exists for); tiles whose 16 rows are equal
reduce to the pinned 1x16 quantizer; the pages' outlier statement on a
constructed tile. The ablation on the single-expert workload's weights
(0.1% outliers of 50x) measures how many nonzero values each scheme flushes
to zero and the relative error of the represented weights.
"""

import numpy as np

from oracle import nvfp4 as Q
from workloads import gen


def _rep(x, rows_per_group=None):
    c, s, o = Q.quantize_tile16(x, rows_per_group)
    return Q.dequantize_tile16(c, s, o, rows_per_group)


def test_transpose_invariance():
    x = gen.normal(41, 0, (64, 96))
    gen.with_outliers(x, 41, 6, frac=0.01)
    c, s, o = Q.quantize_tile16(x)
    ct, st, ot = Q.quantize_tile16(np.ascontiguousarray(x.T))
    assert np.array_equal(Q.unpack_codes(ct), Q.unpack_codes(c).T)
    assert np.array_equal(st, s.T)
    assert np.array_equal(ot, o)
    assert np.array_equal(_rep(np.ascontiguousarray(x.T)), _rep(x).T)


def test_equal_rows_reduce_to_1x16_blocks():
    base = gen.normal(42, 0, (4, 128))
    x = np.repeat(base, 16, axis=0)                     # every tile: 16 equal rows
    x[16:32] *= np.float32(3.0)
    c, s, o = Q.quantize_tile16(x, rows_per_group=32)
    c1, s1, o1 = Q.quantize(x, rows_per_group=32)
    assert np.array_equal(c, c1)
    assert np.array_equal(np.repeat(s, 16, axis=0), s1)
    assert np.array_equal(o, o1)


def test_one_large_value_zeroes_its_tile():
    x = np.full((16, 32), 1.0, dtype=np.float32)
    x[3, 5] = 1000.0
    c, s, o = Q.quantize_tile16(x)
    v = Q.unpack_codes(c)
    assert v[3, 5] == 7                                  # the outlier: E2M1 6.0
    # every other value of the outlier's tile becomes a (positive) zero
    mask = np.zeros((16, 32), bool)
    mask[:, :16] = True
    mask[3, 5] = False
    assert np.all(v[mask] == 0)
    assert np.all(v[:, 16:] != 0)                        # the neighbouring tile keeps its values
    # 1x16 blocks: only the outlier's own block of row 3 is affected
    c1, s1, o1 = Q.quantize(x, rows_per_group=16)
    v1 = Q.unpack_codes(c1)
    assert np.all(v1[np.arange(16) != 3][:, :16] != 0)


def test_ablation_on_single_expert_weights():
    w = gen.single_expert()["w"]                         # [512, 256], 0.1% outliers x50
    nz = w != 0
    t16 = _rep(w)
    c1, s1, o1 = Q.quantize(w, rows_per_group=w.shape[0])
    b16 = Q.dequantize(c1, s1, o1, rows_per_group=w.shape[0])
    flushed_t = int(np.count_nonzero(nz & (t16 == 0)))
    flushed_b = int(np.count_nonzero(nz & (b16 == 0)))
    err = lambda r: float(np.linalg.norm((r - w).astype(np.float64)) / np.linalg.norm(w.astype(np.float64)))
    # the tile scheme flushes several times more values and has the larger error
    assert flushed_t > 3 * flushed_b
    assert err(t16) > 1.2 * err(b16)
