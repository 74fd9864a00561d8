"""GPU parity of the NVFP4 backward against the oracle.

Bit-exact: codes, block scales, outer-scale bits and every stochastic-rounding
outcome of the row-wise quantizer, the transposed re-quantization of saved
activations and weights (both layouts) and of dY, and the padded offsets.
GEMMs (f16 MFMA on exactly dequantized NVFP4 operands): max error 1e-3 of the
group's largest magnitude against the oracle's float64 result on the same
operands, plus the float32 summation bound (L + 3) 2^-24 sum |a b| elementwise.
"""

import numpy as np
import pytest

from helpers import ensure_built, from_dev, to_dev
from oracle import nvfp4 as Q
from oracle import nvfp4_bwd as NB
from oracle import permute as PM
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    ensure_built()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_moe_numerics_nvfp4_amd as nv
    return nv


def _sync():
    import torch
    torch.cuda.synchronize()


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _groups(counts):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return off, NB.padded_offsets(off)


@pytest.mark.parametrize("rows,cols,dtype,case", [
    (300, 1024, "bf16", "outliers"), (64, 256, "f32", "outliers"), (33, 8192, "bf16", "normal"),
    (17, 512, "f32", "tiny_and_zero"),
])
def test_nvfp4_quantize_sr_rows(nv, rows, cols, dtype, case):
    x = gen.normal(401, 0, (rows, cols))
    if case == "outliers":
        gen.with_outliers(x, 401, 6, frac=0.01, factor=50.0)
    if case == "tiny_and_zero":
        x[0] = 0.0
        x[1] *= 1e-30
        x[2, :16] = 0.0
        x[3] *= 1e20
    if dtype == "bf16":
        x = gen.to_bf16_bits(x)
    seed, tag = 0x5EED0401, NB.TAG_DY_ROW
    c, s, o = nv.nvfp4_quantize_sr(to_dev(x), seed, tag)
    _sync()
    rc, rs, ro = NB.quantize_sr_rows(x, seed, tag)
    assert np.array_equal(from_dev(s), rs)
    assert np.array_equal(_bits(from_dev(o)), _bits(ro))
    assert np.array_equal(from_dev(c), rc)


@pytest.mark.parametrize("counts,align", [([5, 0, 300, 128, 1], 128), (list(range(0, 2048, 2)), 128),
                                          ([31, 33], 32), ([], 128)])
def test_moe_padded_offsets(nv, counts, align):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    got = from_dev(nv.moe_padded_offsets(to_dev(off), align))
    _sync()
    assert np.array_equal(got, NB.padded_offsets(off, align))


@pytest.mark.parametrize("counts,cols", [([37, 0, 100, 5, 200], 256), ([64], 128),
                                         ([300, 129], 1024), ([0, 0, 1], 384)])
def test_nvfp4_requant_sr_activations(nv, counts, cols):
    off, poff = _groups(counts)
    M = int(off[-1])
    cap = M + 50
    x = gen.to_bf16_bits(gen.normal(402, 0, (cap, cols)))
    gen_q = Q.quantize(x)
    P = int(poff[-1]) + 128
    seed, tag = 0x5EED0402, NB.TAG_X
    out = nv.nvfp4_requant_sr(*(to_dev(a) for a in gen_q), to_dev(off), to_dev(poff), P, seed, tag)
    _sync()
    rc, rs, ro = NB.requant_sr(*(a[:M] for a in gen_q), off, poff, P, seed, tag)
    pt = int(poff[-1])
    assert np.array_equal(_bits(from_dev(out[2])), _bits(ro))
    assert np.array_equal(from_dev(out[1])[:, :pt // 16], rs[:, :pt // 16])
    assert np.array_equal(from_dev(out[0])[:, :pt // 2], rc[:, :pt // 2])


@pytest.mark.parametrize("E,N,K", [(4, 256, 512), (2, 128, 1024), (8, 512, 256)])
def test_nvfp4_requant_sr_weights_per_expert(nv, E, N, K):
    w = gen.normal(403, 1, (E * N, K), std=0.02)
    gen.with_outliers(w, 403, 7)
    w = gen.to_bf16_bits(w)
    wq = Q.quantize(w, rows_per_group=N)
    woff = np.arange(E + 1, dtype=np.int64) * N
    seed, tag = 0x5EED0403, NB.TAG_W
    out = nv.nvfp4_requant_sr(*(to_dev(a) for a in wq), to_dev(woff), to_dev(woff), E * N, seed,
                              tag, rows_per_group=N, per_group_layout=True)
    _sync()
    rc, rs, ro = NB.requant_weights_sr(*wq, E, seed, tag)
    assert np.array_equal(_bits(from_dev(out[2])), _bits(ro))
    assert np.array_equal(from_dev(out[1]), rs)
    assert np.array_equal(from_dev(out[0]), rc)


@pytest.mark.parametrize("counts,cols,dtype", [([37, 0, 100, 5, 200], 256, "bf16"),
                                               ([300, 129], 1024, "f32"), ([128], 128, "bf16")])
def test_nvfp4_quantize_sr_colwise(nv, counts, cols, dtype):
    off, poff = _groups(counts)
    M = int(off[-1])
    dy = gen.normal(404, 3, (M, cols), std=1e-3)
    if dtype == "bf16":
        dy = gen.to_bf16_bits(dy)
    P = int(poff[-1])
    seed, tag = 0x5EED0404, NB.TAG_DY_COL
    out = nv.nvfp4_quantize_sr_colwise(to_dev(dy), to_dev(off), to_dev(poff), P, seed, tag)
    _sync()
    rc, rs, ro = NB.quantize_sr_grouped_T(Q._as_f32(dy), off, poff, P, seed, tag)
    assert np.array_equal(_bits(from_dev(out[2])), _bits(ro))
    assert np.array_equal(from_dev(out[1]), rs)
    assert np.array_equal(from_dev(out[0]), rc)


def _gemm_check(got, ref64, absmag, L, what):
    d = np.abs(got.astype(np.float64) - ref64)
    m = np.abs(ref64).max()
    assert d.max() <= 1e-3 * m + 1e-30, f"{what}: normwise {d.max() / max(m, 1e-300):.3e}"
    bound = (L + 3) * 2.0 ** -24 * absmag
    assert np.all(d <= bound * 1.0000001 + 1e-37), f"{what}: summation bound"


@pytest.mark.parametrize("counts,N,K", [([37, 0, 300, 128], 256, 512), ([1000], 512, 256),
                                        ([5, 260, 0, 90, 700], 256, 256)])
def test_wgrad_nvfp4(nv, counts, N, K):
    off, poff = _groups(counts)
    M = int(off[-1])
    P = int(poff[-1])
    dy = gen.normal(405, 3, (M, N), std=1e-3)
    x = gen.normal(405, 0, (M, K))
    gen.with_outliers(x, 405, 6, frac=0.01)
    dyT = NB.quantize_sr_grouped_T(dy, off, poff, P, 1, NB.TAG_DY_COL)
    xT = NB.quantize_sr_grouped_T(x, off, poff, P, 1, NB.TAG_X)
    dw = nv.moe_bwd_wgrad_nvfp4(tuple(to_dev(a) for a in dyT), tuple(to_dev(a) for a in xT),
                                to_dev(poff), N, K)
    _sync()
    got = from_dev(dw)
    ref = NB.wgrad(dyT, xT, poff, accum="fp64")
    A = np.abs(Q.dequantize(dyT[0], dyT[1], None, apply_outer=False).astype(np.float64))
    B = np.abs(Q.dequantize(xT[0], xT[1], None, apply_outer=False).astype(np.float64))
    for g in range(len(counts)):
        a, b = int(poff[g]), int(poff[g + 1])
        if b == a:
            assert np.all(got[g] == 0)
            continue
        mag = (A[:, a:b] @ B[:, a:b].T) * float(dyT[2][g]) * float(xT[2][g])
        _gemm_check(got[g], ref[g], mag, b - a, f"wgrad group {g}")


@pytest.mark.parametrize("counts,N,K", [([37, 0, 300, 128], 256, 512), ([900, 11], 1024, 256)])
def test_dgrad_nvfp4_through_forward_gemm(nv, counts, N, K):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    E = len(counts)
    M = int(off[-1])
    dy = gen.to_bf16_bits(gen.normal(406, 3, (M, N), std=1e-3))
    w = gen.to_bf16_bits(gen.normal(406, 1, (E * N, K), std=0.02))
    dyq = NB.quantize_sr_rows(dy, 2)
    wT = NB.requant_weights_sr(*Q.quantize(w, rows_per_group=N), E, seed=2)
    dx = nv.moe_fwd_grouped_gemm(*(to_dev(a) for a in dyq), *(to_dev(a) for a in wT), to_dev(off))
    _sync()
    got = from_dev(dx)[:M]
    ref = NB.dgrad(dyq, wT, off, K, accum="fp64")
    A = np.abs(Q.dequantize(dyq[0], dyq[1], None, apply_outer=False).astype(np.float64))
    B = np.abs(Q.dequantize(wT[0], wT[1], None, apply_outer=False).astype(np.float64))
    for g in range(E):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        mag = (A[a:b] @ B[g * K:(g + 1) * K].T) * dyq[2][a:b, None] * float(wT[2][g])
        _gemm_check(got[a:b], ref[a:b], mag, N, f"dgrad group {g}")
