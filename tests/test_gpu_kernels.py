"""GPU parity of every entry point against the oracle, at sizes the oracle
finishes in seconds that still span several tiles and a ragged tail.

Bit-exact: NVFP4 codes, block scales, outer-scale float bits, permutation
indices and offsets, gathered rows, MXFP8 elements and E8M0 scales (including
every stochastic-rounding outcome). GEMMs: max relative error 1e-3 per group
(normwise) against the oracle's float64 result on the same quantized
operands, plus an elementwise summation-error bound; an exact-arithmetic case
must match bit for bit.

* Forward (f16 MFMA on exactly dequantized operands): also elementwise
  relative error 1e-3 on the non-tiny entries, and the float32 bound
  (K + 3) * 2^-24 * sum|a*b| that any float32 accumulation order satisfies.
* dgrad / wgrad (block-scaled FP8 MFMA): measured on gfx950, that
  instruction forms each 32-element MX block's dot product by aligning the 32
  exact products to the block's largest one and dropping bits 14 or more
  binades below it (a 448*448 product absorbs a 4.5 product; a lone product,
  or products of different blocks, are exact), then adds the scaled block sums
  in float32. Its elementwise bound is therefore
  sum over blocks of 31 * 2^-13 * max_block|a*b| (2x margin on the dropped
  bits) plus the float32 bound; the elementwise relative check is not applied
  to these two, the 1e-3 normwise contract is.
"""

import numpy as np
import pytest

from helpers import assert_gemm_close, ensure_built, from_dev, to_dev, w8_blocked
from oracle import ffn as FF
from oracle import formats as F
from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
from oracle import permute as PM
from workloads import gen

pytestmark = pytest.mark.gpu



def mx_bound(Aabs, Babs):
    """Elementwise error bound of C = A @ B^T on the block-scaled FP8 MFMA for
    |A| [R, L], |B| [C, L] (float64, L a multiple of 32): the per-block
    alignment loss plus the float32 summation bound."""
    R, L = Aabs.shape
    out = (L + 3) * 2.0 ** -24 * (Aabs @ Babs.T)
    for j in range(0, L, 32):
        m = np.max(Aabs[:, None, j:j + 32] * Babs[None, :, j:j + 32], axis=2)
        out += 31 * 2.0 ** -13 * m
    return out


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


# ------------------------------------------------------------------ quantize

def _quant_input(seed, rows, cols, bf16):
    x = gen.normal(seed, 0, (rows, cols))
    gen.with_outliers(x, seed, 6, frac=0.01)
    if rows > 3:
        x[rows // 2] = 0.0                       # zero row
        x[1] *= np.float32(1e-20)                # tiny row (still normal range)
        x[2, 16:32] = 0.0                        # zero block
        x[2, 17] = -0.0
        x[3, :] = np.float32(1e4)                # constant row
    return gen.to_bf16_bits(x) if bf16 else x


@pytest.mark.parametrize("bf16,rows,cols", [
    (False, 64, 256), (True, 257, 1024), (True, 33, 4096), (True, 5, 2048),
    (False, 7, 8192), (True, 1, 32), (True, 100, 96), (False, 130, 1536),
])
def test_nvfp4_quantize_per_token(nv, bf16, rows, cols):
    a = _quant_input(1000 + rows + cols, rows, cols, bf16)
    c, s, o = nv.nvfp4_quantize(to_dev(a))
    _sync()
    rc, rs, ro = Q.quantize(a)
    assert np.array_equal(from_dev(c), rc)
    assert np.array_equal(from_dev(s), rs)
    assert np.array_equal(_bits(from_dev(o)), _bits(ro))


def test_nvfp4_quantize_bruteforce_codes_and_scales(nv):
    """Rows built from every E2M1 code times every E4M3 scale, with and
    without a perturbation of 1 ulp, and values that land near every E2M1
    midpoint after scaling."""
    rows = []
    base = np.arange(16)
    for s_code in range(1, 0x7F):
        S = F.e4m3_decode(s_code)
        v = (F.e2m1_decode(base) * S).astype(np.float32)
        rows.append(v)
        rows.append(np.nextafter(v, np.float32(np.inf)).astype(np.float32))
        rows.append(np.nextafter(v, np.float32(-np.inf)).astype(np.float32))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    for j in range(-20, 21, 3):
        sc = np.float32(2.0 ** j)
        row = np.concatenate([mids, -mids]).astype(np.float32) * sc
        rows.append(row)
    x = np.stack(rows).astype(np.float32)
    x = np.concatenate([x, x], axis=1)                 # 32 columns
    c, s, o = nv.nvfp4_quantize(to_dev(x))
    _sync()
    rc, rs, ro = Q.quantize(x)
    assert np.array_equal(from_dev(c), rc)
    assert np.array_equal(from_dev(s), rs)
    assert np.array_equal(_bits(from_dev(o)), _bits(ro))


@pytest.mark.parametrize("bf16,E,N,K", [(True, 3, 64, 256), (False, 1, 512, 256), (True, 8, 32, 1024)])
def test_nvfp4_quantize_per_expert(nv, bf16, E, N, K):
    w = gen.normal(77 + E, 1, (E * N, K), std=0.02)
    gen.with_outliers(w, 77 + E, 7, frac=0.001)
    if E > 2:
        w[N:2 * N] = 0.0                               # an all-zero expert
    a = gen.to_bf16_bits(w) if bf16 else w
    c, s, o = nv.nvfp4_quantize(to_dev(a), rows_per_group=N)
    _sync()
    rc, rs, ro = Q.quantize(a, rows_per_group=N)
    assert np.array_equal(from_dev(c), rc)
    assert np.array_equal(from_dev(s), rs)
    assert np.array_equal(_bits(from_dev(o)), _bits(ro))


@pytest.mark.parametrize("bf16,rows,cols,rpg", [(True, 512, 256, None), (False, 64, 96, 32),
                                                 (True, 4096, 1024, 512), (True, 48, 4112, 16)])
def test_nvfp4_quantize_tile16(nv, bf16, rows, cols, rpg):
    x = gen.normal(450 + rows, 0, (rows, cols))
    gen.with_outliers(x, 450 + rows, 6, frac=0.001)
    x[:16, :16] = 0.0                                        # a zero tile
    if rows >= 64:
        x[32:48] *= np.float32(1e-30)                        # tiny values (zero tiles for rpg 16..32)
    a = gen.to_bf16_bits(x) if bf16 else x
    c, sc, o = nv.nvfp4_quantize_tile16(to_dev(a), rows_per_group=rpg)
    _sync()
    rc, rs, ro = Q.quantize_tile16(a, rows_per_group=rpg)
    assert np.array_equal(from_dev(c), rc)
    assert np.array_equal(from_dev(sc), rs)
    assert np.array_equal(_bits(from_dev(o)), _bits(ro))


# ------------------------------------------------------------------ permute

# up to 16384 routed pairs take the one-launch form, more the three-launch one;
# K = 96 and 160 copy the scale rows bytewise, K = 256 in 16-byte pieces
@pytest.mark.parametrize("case,K", [("uniform", 256), ("zipf", 256), ("one_expert", 256),
                                    ("none_local", 256), ("single", 256), ("empty", 256),
                                    ("many_experts", 256), ("uniform", 160), ("zipf", 96),
                                    ("zipf_many", 256), ("above_small", 256),
                                    ("one_local_big", 128)])
def test_moe_permute(nv, case, K):
    import torch
    if case == "uniform":
        topk, e0, nl = gen.route_uniform(201, 1000, 64, 8), 16, 8
    elif case == "zipf":
        topk, e0, nl = gen.route_zipf(202, 3000, k=8, n_experts=384), 144, 48
    elif case == "one_expert":
        topk, e0, nl = np.full((700, 1), 5, np.int32), 0, 8
    elif case == "none_local":
        topk, e0, nl = gen.route_uniform(203, 50, 16, 2), 100, 4
    elif case == "zipf_many":          # three-launch form with 1024 local experts
        topk, e0, nl = gen.route_zipf(206, 2500, k=8, n_experts=2048), 512, 1024
    elif case == "many_experts":       # the largest local expert count, 1024
        topk, e0, nl = gen.route_uniform(205, 900, 1024, 4), 0, 1024
    elif case == "single":
        topk, e0, nl = np.zeros((64, 1), np.int32), 0, 1
    elif case == "above_small":        # 16640 pairs: three-launch form, 8 local experts
        topk, e0, nl = gen.route_uniform(207, 8320, 8, 2), 0, 8
    elif case == "one_local_big":      # 16385 pairs over one local expert
        topk, e0, nl = gen.route_uniform(208, 16385, 4, 1), 2, 1
    else:
        topk, e0, nl = np.zeros((0, 2), np.int32), 0, 4
    T, k = topk.shape
    x = gen.to_bf16_bits(gen.normal(204, 0, (max(T, 1), K)))[:T]
    xc, xs, xo = Q.quantize(x) if T else (np.zeros((0, K // 2), np.uint8),
                                          np.zeros((0, K // 16), np.uint8),
                                          np.zeros((0,), np.float32))
    o = nv.moe_permute(to_dev(topk) if T else torch.zeros((0, k), dtype=torch.int32, device="cuda"),
                       e0, nl,
                       to_dev(xc) if T else torch.zeros((0, K // 2), dtype=torch.uint8, device="cuda"),
                       to_dev(xs) if T else torch.zeros((0, K // 16), dtype=torch.uint8, device="cuda"),
                       to_dev(xo) if T else torch.zeros((0,), dtype=torch.float32, device="cuda"))
    _sync()
    off, pad, rt, rs = PM.permute(topk, e0, nl)
    M = int(off[-1])
    assert np.array_equal(from_dev(o["offsets"]), off)
    assert np.array_equal(from_dev(o["padded_offsets"]), pad)
    assert np.array_equal(from_dev(o["row_token"])[:M], rt)
    assert np.array_equal(from_dev(o["row_slot"])[:M], rs)
    if T:
        assert np.array_equal(from_dev(o["pair_row"]), FF.pair_rows(topk, e0, nl))
    if M:
        gc, gs, go = PM.gather_rows(rt, xc, xs, xo)
        assert np.array_equal(from_dev(o["codes"])[:M], gc)
        assert np.array_equal(from_dev(o["scales"])[:M], gs)
        assert np.array_equal(_bits(from_dev(o["outer"])[:M]), _bits(go))


# ------------------------------------------------------------------ requant

def _groups_from_counts(counts):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return off, MX.padded_offsets_from_offsets(off)


@pytest.mark.parametrize("counts,cols", [
    ([37, 0, 100, 5, 200], 256), ([64], 128), ([1, 2, 3], 384), ([300, 129], 1024),
])
def test_requant_sr_activations(nv, counts, cols):
    import torch
    off, pad = _groups_from_counts(counts)
    M = int(off[-1])
    x = gen.normal(300 + cols, 0, (M, cols))
    gen.with_outliers(x, 300 + cols, 6, frac=0.01)
    x[min(3, M - 1)] = 0.0
    if len(counts) > 2:
        # a whole group of tiny rows: outer scales near the bottom of float32,
        # so its 32-token blocks take E8M0 codes down to 0 (2^-127)
        x[off[2]:off[3]] *= np.float32(1e-37)
    qc, qs, qo = Q.quantize(gen.to_bf16_bits(x))
    P = int(pad[-1]) + 64                                  # extra columns stay untouched
    seed, tag = 0x5EED0004, 0
    out = torch.full((cols, P), 0xCD, dtype=torch.uint8, device="cuda")
    out_e8 = torch.full((cols, P // 32), 0xCD, dtype=torch.uint8, device="cuda")
    nv.mxfp8_requant_sr(to_dev(qc), to_dev(qs), to_dev(qo), to_dev(off), to_dev(pad), P, seed, tag,
                        out=out, out_e8=out_e8)
    _sync()
    rq, re = MX.requant_sr(qc, qs, qo, off, pad, P, seed, tag)
    pt = int(pad[-1])
    got, got_e = from_dev(out), from_dev(out_e8)
    assert np.array_equal(got[:, :pt], rq[:, :pt])
    assert np.array_equal(got_e[:, :pt // 32], re[:, :pt // 32])
    assert np.all(got[:, pt:] == 0xCD) and np.all(got_e[:, pt // 32:] == 0xCD)
    # deterministic across calls
    out2, e2 = nv.mxfp8_requant_sr(to_dev(qc), to_dev(qs), to_dev(qo), to_dev(off), to_dev(pad), P,
                                   seed, tag)
    _sync()
    assert np.array_equal(from_dev(out2)[:, :pt], got[:, :pt])


@pytest.mark.parametrize("E,N,K", [(1, 512, 256), (4, 96, 384), (8, 256, 128)])
def test_requant_sr_weights(nv, E, N, K):
    w = gen.to_bf16_bits(gen.normal(400 + E, 1, (E * N, K), std=0.02))
    qc, qs, qo = Q.quantize(w, rows_per_group=N)
    off = np.arange(E + 1, dtype=np.int64) * N
    seed, tag = 0x5EED0002, 1
    out, oe = nv.mxfp8_requant_sr(to_dev(qc), to_dev(qs), to_dev(qo), to_dev(off), to_dev(off),
                                  E * N, seed, tag, rows_per_group=N)
    _sync()
    rq, re = MX.requant_sr(qc, qs, qo, off, off, E * N, seed, tag, rows_per_group=N)
    # the library stores each expert's transposed block [K, N] contiguously:
    # the oracle's [K, E*N] values, rearranged
    assert from_dev(out).shape == (E * K, N)
    assert np.array_equal(from_dev(out), w8_blocked(rq, E))
    assert np.array_equal(from_dev(oe), w8_blocked(re, E))


def test_requant_sr_per_group_blocks_uneven(nv):
    """The per-group (weight) mode through the C ABI with transpose groups of
    different padded lengths (64, 160, 96) and short groups: group g's block
    [cols, L_g] starts at element cols * padded[g], its E8M0 bytes at
    cols * padded[g] / 32, and every byte equals the oracle's [cols, P]
    result at the same (column, padded position), padding zeros included."""
    import torch
    from precision_moe_numerics_nvfp4_amd import binding as B
    rows, cols, rpg = 256, 256, 64
    w = gen.to_bf16_bits(gen.normal(470, 1, (rows, cols), std=0.02))
    qc, qs, qo = Q.quantize(w, rows_per_group=rpg)
    off = np.array([0, 40, 170, 256], dtype=np.int64)
    pad = np.array([0, 64, 224, 320], dtype=np.int64)
    P, G, seed, tag = 320, 3, 0x5EED0007, 1
    out = torch.full((cols * P,), 0xCD, dtype=torch.uint8, device="cuda")
    oe = torch.full((cols * P // 32,), 0xCD, dtype=torch.uint8, device="cuda")
    dc, ds, do, doff, dpad = to_dev(qc), to_dev(qs), to_dev(qo), to_dev(off), to_dev(pad)
    st = B.lib().mxfp8_requant_sr(B._ptr(dc), B._ptr(ds), B._ptr(do), 1, rpg, rows, cols,
                                  B._ptr(doff), B._ptr(dpad), G, P, seed, tag, B._ptr(out),
                                  B._ptr(oe), B._stream(dc))
    assert st == 0
    _sync()
    rq, re = MX.requant_sr(qc, qs, qo, off, pad, P, seed, tag, rows_per_group=rpg)
    want_q = np.concatenate([rq[:, pad[g]:pad[g + 1]].reshape(-1) for g in range(G)])
    want_e = np.concatenate([re[:, pad[g] // 32:pad[g + 1] // 32].reshape(-1) for g in range(G)])
    assert np.array_equal(from_dev(out), want_q)
    assert np.array_equal(from_dev(oe), want_e)


# ------------------------------------------------------------------ dY quantize

@pytest.mark.parametrize("bf16,rows,cols", [(True, 100, 256), (False, 64, 512), (True, 1, 32), (True, 513, 2048)])
def test_mxfp8_quantize_rowwise(nv, bf16, rows, cols):
    x = gen.normal(500 + rows, 3, (rows, cols), std=1e-3)
    x[0, :32] = 0.0
    x[-1, -32:] *= np.float32(1e-30)
    a = gen.to_bf16_bits(x) if bf16 else x
    q, e = nv.mxfp8_quantize(to_dev(a), "rowwise")
    _sync()
    rq, re = MX.quantize_rowwise(a)
    assert np.array_equal(from_dev(q), rq)
    assert np.array_equal(from_dev(e), re)


@pytest.mark.parametrize("bf16,counts,cols", [(True, [37, 0, 100, 5], 256), (False, [64, 65], 512),
                                              (True, [1000], 128), (False, [40, 3, 70], 256)])
def test_mxfp8_quantize_colwise(nv, bf16, counts, cols):
    off, pad = _groups_from_counts(counts)
    M = int(off[-1])
    x = gen.normal(600 + cols, 3, (M, cols), std=1e-3)
    if len(counts) > 2:
        x[off[2]:off[3]] *= np.float32(1e-36)   # blocks with E8M0 codes near 0, subnormal inputs
    a = gen.to_bf16_bits(x) if bf16 else x
    P = int(pad[-1])
    q, e = nv.mxfp8_quantize(to_dev(a), "colwise", to_dev(off), to_dev(pad), P)
    _sync()
    rq, re = MX.quantize_colwise_grouped(a, off, pad, P)
    assert np.array_equal(from_dev(q), rq)
    assert np.array_equal(from_dev(e), re)


@pytest.mark.parametrize("bf16,counts,cols", [(True, [37, 0, 100, 5], 256), (False, [64, 65], 512),
                                              (True, [1000, 3], 128), (False, [40, 3, 70], 256)])
def test_mxfp8_quantize_dual(nv, bf16, counts, cols):
    import torch
    off, pad = _groups_from_counts(counts)
    M = int(off[-1])
    x = gen.normal(650 + cols, 3, (M + 5, cols), std=1e-3)    # 5 rows past the groups
    if len(counts) > 2:
        x[off[2]:off[3]] *= np.float32(1e-36)
    a = gen.to_bf16_bits(x) if bf16 else x
    P = int(pad[-1]) + 32
    row = (torch.full((M + 5, cols), 0xCD, dtype=torch.uint8, device="cuda"),
           torch.full((M + 5, cols // 32), 0xCD, dtype=torch.uint8, device="cuda"))
    rq, re_, cq, ce = nv.mxfp8_quantize_dual(to_dev(a), to_dev(off), to_dev(pad), P, row_out=row)
    _sync()
    wr, wre = MX.quantize_rowwise(a[:M])
    wc, wce = MX.quantize_colwise_grouped(a[:M], off, pad, P)
    assert np.array_equal(from_dev(rq)[:M], wr)
    assert np.array_equal(from_dev(re_)[:M], wre)
    assert np.all(from_dev(rq)[M:] == 0xCD) and np.all(from_dev(re_)[M:] == 0xCD)
    pt = int(pad[-1])
    assert np.array_equal(from_dev(cq)[:, :pt], wc[:, :pt])
    assert np.array_equal(from_dev(ce)[:, :pt // 32], wce[:, :pt // 32])


# ------------------------------------------------------------------ forward GEMM

def _fwd_case(seed, T, K, N, E, k, exact=False):
    case = gen.moe_case(seed, T=T, K=K, N=N, E=E, k=k)
    xc, xs, xo = Q.quantize(case["x"])
    wc, ws, wo = Q.quantize(case["w"], rows_per_group=N)
    if exact:
        # narrow block scales and power-of-two outer scales: every partial sum
        # is exact in float32, so any summation order gives the same bits
        xs[:] = np.where(xs > 0, 0x38 + (xs & 1), 0).astype(np.uint8)
        ws[:] = np.where(ws > 0, 0x38 + (ws & 1), 0).astype(np.uint8)
        xo[:] = np.ldexp(np.float32(1), (np.arange(xo.size) % 7 - 3).astype(np.int32))
        wo[:] = np.ldexp(np.float32(1), (np.arange(wo.size) % 5 - 2).astype(np.int32))
    off, pad, rt, rs = PM.permute(case["topk"], 0, E)
    ac, asc, ao = PM.gather_rows(rt, xc, xs, xo)
    return ac, asc, ao, wc, ws, wo, off


def _fwd_bound(ac, asc, ao, wc, ws, wo, off, N, K):
    A = np.abs(Q.dequantize(ac, asc, None, apply_outer=False)).astype(np.float64)
    G = wo.size
    B = np.abs(Q.dequantize(wc, ws, None, apply_outer=False)).astype(np.float64).reshape(G, N, K)
    out = np.zeros((A.shape[0], N))
    for g in range(G):
        a, b = off[g], off[g + 1]
        out[a:b] = (A[a:b] @ B[g].T) * np.abs(ao[a:b, None]) * abs(float(wo[g]))
    return (K + 3) * 2.0 ** -24 * out


@pytest.mark.parametrize("T,K,N,E,k", [(300, 512, 256, 4, 2), (64, 256, 512, 1, 1), (500, 384, 384, 6, 3),
                                         # 256-row tiles: one K stage; several m- and n-tiles, ragged ends
                                         (700, 128, 512, 3, 2), (1000, 1024, 256, 2, 1),
                                         # few rows per expert (weight streaming): one and two
                                         # 16-row blocks per expert, one or three K chunks per wave
                                         (100, 512, 256, 16, 2), (60, 1536, 128, 8, 4)])
def test_fwd_grouped_gemm(nv, T, K, N, E, k):
    import torch
    ac, asc, ao, wc, ws, wo, off = _fwd_case(700 + T, T, K, N, E, k)
    M = int(off[-1])
    cap = M + 40                                              # rows past M stay untouched
    dac = torch.zeros((cap, K // 2), dtype=torch.uint8, device="cuda")
    dac[:M] = to_dev(ac)
    das = torch.zeros((cap, K // 16), dtype=torch.uint8, device="cuda")
    das[:M] = to_dev(asc)
    dao = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    dao[:M] = to_dev(ao)
    y = torch.full((cap, N), float("nan"), dtype=torch.float32, device="cuda")
    nv.moe_fwd_grouped_gemm(dac, das, dao, to_dev(wc), to_dev(ws), to_dev(wo), to_dev(off), y=y)
    _sync()
    got = from_dev(y)
    assert np.all(np.isnan(got[M:]))
    ref = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, N, accum="fp64")
    groups = [(off[g], off[g + 1]) for g in range(E)]
    assert_gemm_close(got[:M], ref, groups, _fwd_bound(ac, asc, ao, wc, ws, wo, off, N, K), what="fwd")
    # bf16 output: within one bf16 step of the exact value
    yb = nv.moe_fwd_grouped_gemm(dac, das, dao, to_dev(wc), to_dev(ws), to_dev(wo), to_dev(off),
                                 out_dtype=torch.bfloat16)
    _sync()
    gb = F.bf16_bits_to_f32(from_dev(yb)[:M]).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    assert np.all(np.abs(gb - ref) <= ulp * 1.0000001)


def _fwd_counts_case(seed, counts, K, N):
    """Expert groups of the given row counts (routed rows already grouped)."""
    M, E = int(sum(counts)), len(counts)
    xc, xs, xo = Q.quantize(gen.to_bf16_bits(gen.normal(seed, 0, (max(M, 1), K))))
    wc, ws, wo = Q.quantize(gen.to_bf16_bits(gen.normal(seed, 1, (E * N, K), std=0.02)),
                            rows_per_group=N)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return xc[:M], xs[:M], xo[:M], wc, ws, wo, off


# Groups whose row count is just past a multiple of 256 (tails of 5, 32, 31,
# 33, 44, 1, 128 rows, larger partial tiles of 129 and 200 rows, whole
# groups of 20 and 100 rows): with at most one round of workgroups every tail
# is a partial 256-row tile. The last case has 300 tiles of 256 x 256 on
# MI355X's 256 compute units, 100 of them full: its 200 tails (44 and 100
# rows) run in the weight-streaming kernel after one round of full tiles.
@pytest.mark.parametrize("counts,K,N", [([261, 544, 33, 20, 256, 0, 300, 287], 1024, 512),
                                        ([261, 544, 33, 20, 256, 0, 300, 287], 384, 256),
                                        ([257, 288, 300], 1536, 256),
                                        ([384, 385, 100, 0, 456, 1037], 512, 768),
                                        ([300, 100] * 100, 512, 256)])
def test_fwd_grouped_gemm_tails(nv, counts, K, N):
    import torch
    ac, asc, ao, wc, ws, wo, off = _fwd_counts_case(800 + K, counts, K, N)
    M = int(off[-1])
    cap = M + 8                                               # rows past M stay untouched
    dac = torch.zeros((cap, K // 2), dtype=torch.uint8, device="cuda")
    dac[:M] = to_dev(ac)
    das = torch.zeros((cap, K // 16), dtype=torch.uint8, device="cuda")
    das[:M] = to_dev(asc)
    dao = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    dao[:M] = to_dev(ao)
    y = torch.full((cap, N), float("nan"), dtype=torch.float32, device="cuda")
    nv.moe_fwd_grouped_gemm(dac, das, dao, to_dev(wc), to_dev(ws), to_dev(wo), to_dev(off), y=y)
    _sync()
    got = from_dev(y)
    assert np.all(np.isnan(got[M:]))
    ref = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, N, accum="fp64")
    groups = [(off[g], off[g + 1]) for g in range(len(counts))]
    assert_gemm_close(got[:M], ref, groups, _fwd_bound(ac, asc, ao, wc, ws, wo, off, N, K), what="fwd")


def test_fwd_grouped_gemm_exact_case(nv):
    ac, asc, ao, wc, ws, wo, off = _fwd_case(731, 200, 256, 256, 3, 2, exact=True)
    y = nv.moe_fwd_grouped_gemm(to_dev(ac), to_dev(asc), to_dev(ao), to_dev(wc), to_dev(ws),
                                to_dev(wo), to_dev(off))
    _sync()
    r32 = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, 256)
    r64 = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, 256, accum="fp64")
    assert np.array_equal(r32.astype(np.float64), r64)       # the case is exact
    assert np.array_equal(from_dev(y), r32)


# ------------------------------------------------------------------ backward GEMMs

def _mx(x):
    return MX.quantize_rne(np.asarray(x, np.float32))


# 128-row tiles (few rows per group); 256 x 128 tiles (256-row tiles that
# would not fill the chip: ragged groups, an empty one, a 32-row contraction
# tail); 256 x 256 tiles (a large capacity)
# Tile paths: 128 x 128 (the first three), 320 x 128 (about one round of
# them covers the output: the next three), 256 x 256 (the last).
@pytest.mark.parametrize("counts,N,K,extra", [([100, 0, 37, 250], 256, 384, 33), ([64], 512, 256, 33),
                                              ([129, 3], 128, 128, 33),
                                              ([300, 700, 0, 600], 512, 256, 33),
                                              ([1000, 24], 256, 512, 8000),
                                              ([1037, 1018, 992, 1068], 512, 1024, 5),
                                              ([2000, 1500, 900], 256, 4096, 33)])
def test_dgrad(nv, counts, N, K, extra):
    import torch
    off, pad = _groups_from_counts(counts)
    M, G = int(off[-1]), len(counts)
    dy = gen.normal(800 + N, 3, (M, N), std=1e-3)
    wT = gen.normal(801 + N, 1, (K, G * N), std=0.02)
    dq, de = _mx(dy)
    wq, we = _mx(wT)
    cap = M + extra
    ddq = torch.zeros((cap, N), dtype=torch.uint8, device="cuda")
    ddq[:M] = to_dev(dq)
    dde = torch.zeros((cap, N // 32), dtype=torch.uint8, device="cuda")
    dde[:M] = to_dev(de)
    dx = torch.full((cap, K), float("nan"), dtype=torch.float32, device="cuda")
    nv.moe_bwd_dgrad(ddq, dde, to_dev(w8_blocked(wq, G)), to_dev(w8_blocked(we, G)), to_dev(off), N,
                     K, dx=dx)
    _sync()
    got = from_dev(dx)
    assert np.all(np.isnan(got[M:]))
    ref = GM.dgrad_grouped(dq, de, wq, we, off, N, accum="fp64")
    DY, W = np.abs(MX.dequantize(dq, de)), np.abs(MX.dequantize(wq, we))
    bound = np.zeros((M, K))
    for g in range(G):
        bound[off[g]:off[g + 1]] = mx_bound(DY[off[g]:off[g + 1]], W[:, g * N:(g + 1) * N])
    groups = [(off[g], off[g + 1]) for g in range(G)]
    assert_gemm_close(got[:M], ref, groups, bound, what="dgrad", elementwise=False)


# all-MXFP8 forward: 256x256 tiles (m_cap >= 256 G, N % 256 == 0) and the
# 128-row fallback, ragged groups, an empty group
@pytest.mark.parametrize("counts,N,K", [([300, 0, 517, 260], 512, 384), ([1100], 256, 1024),
                                        ([37, 5, 100], 384, 256), ([64, 200], 128, 640)])
def test_fwd_grouped_gemm_mxfp8(nv, counts, N, K):
    import torch
    off, pad = _groups_from_counts(counts)
    M, G = int(off[-1]), len(counts)
    x = gen.normal(900 + N, 0, (M, K))
    gen.with_outliers(x, 900 + N, 6, frac=0.01)
    w = gen.normal(901 + N, 1, (G * N, K), std=0.02)
    xq, xe = _mx(x)
    wq, we = _mx(w)
    cap = M + 19
    dxq = torch.zeros((cap, K), dtype=torch.uint8, device="cuda")
    dxq[:M] = to_dev(xq)
    dxe = torch.zeros((cap, K // 32), dtype=torch.uint8, device="cuda")
    dxe[:M] = to_dev(xe)
    y = torch.full((cap, N), float("nan"), dtype=torch.float32, device="cuda")
    nv.moe_fwd_grouped_gemm_mxfp8(dxq, dxe, to_dev(wq), to_dev(we), to_dev(off), y=y)
    _sync()
    got = from_dev(y)
    assert np.all(np.isnan(got[M:]))
    ref = GM.fwd_grouped_mxfp8(xq, xe, wq, we, off, N, accum="fp64")
    X, W = np.abs(MX.dequantize(xq, xe)), np.abs(MX.dequantize(wq, we)).reshape(G, N, K)
    bound = np.zeros((M, N))
    for g in range(G):
        bound[off[g]:off[g + 1]] = mx_bound(X[off[g]:off[g + 1]], W[g])
    groups = [(off[g], off[g + 1]) for g in range(G)]
    assert_gemm_close(got[:M], ref, groups, bound, what="fwd mxfp8", elementwise=False)
    # bf16 output: within one bf16 step of the exact value where the float32
    # result is within its bound
    yb = nv.moe_fwd_grouped_gemm_mxfp8(dxq, dxe, to_dev(wq), to_dev(we), to_dev(off),
                                       out_dtype=torch.bfloat16)
    _sync()
    gb = F.bf16_bits_to_f32(from_dev(yb)[:M]).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    assert np.all(np.abs(gb - ref) <= ulp * 1.0000001 + bound)


def test_mxfp8_gather_rows(nv):
    import torch
    topk, e0, nl = gen.route_uniform(905, 700, 16, 3), 4, 8
    T, k = topk.shape
    K = 288
    x8, xe = _mx(gen.normal(906, 0, (T, K)))
    o = nv.moe_permute(to_dev(topk), e0, nl,
                       *(to_dev(a) for a in Q.quantize(gen.to_bf16_bits(gen.normal(907, 0, (T, 256))))))
    _sync()
    off, pad, rt, rs = PM.permute(topk, e0, nl)
    M = int(off[-1])
    cap = T * k
    dq = torch.full((cap, K), 0xAB, dtype=torch.uint8, device="cuda")
    de = torch.full((cap, K // 32), 0xAB, dtype=torch.uint8, device="cuda")
    nv.mxfp8_gather_rows(o["row_token"], o["offsets"], to_dev(x8), to_dev(xe), out=(dq, de))
    _sync()
    assert np.array_equal(from_dev(dq)[:M], x8[rt])
    assert np.array_equal(from_dev(de)[:M], xe[rt])
    assert np.all(from_dev(dq)[M:] == 0xAB) and np.all(from_dev(de)[M:] == 0xAB)


@pytest.mark.parametrize("counts,N,K", [([100, 0, 37, 250], 256, 384), ([64], 512, 256), ([129, 3], 128, 128),
                                         # unsorted sizes with ties (tiles are ranked by size)
                                         ([40, 300, 0, 40, 130, 300, 7], 256, 512)])
def test_wgrad(nv, counts, N, K):
    off, pad = _groups_from_counts(counts)
    G = len(counts)
    P = int(pad[-1])
    dy = gen.normal(900 + N, 3, (int(off[-1]), N), std=1e-3)
    x = gen.normal(901 + N, 0, (int(off[-1]), K))
    dyq, dye = MX.quantize_colwise_grouped(dy, off, pad, P)
    xq, xe = MX.quantize_colwise_grouped(x, off, pad, P)
    dw = nv.moe_bwd_wgrad(to_dev(dyq), to_dev(dye), to_dev(xq), to_dev(xe), to_dev(pad), N, K)
    _sync()
    got = from_dev(dw)
    ref = GM.wgrad_grouped(dyq, dye, xq, xe, pad, accum="fp64")
    DY, X = np.abs(MX.dequantize(dyq, dye)), np.abs(MX.dequantize(xq, xe))
    for g in range(G):
        a, b = pad[g], pad[g + 1]
        if b == a:
            assert np.all(got[g] == 0)
            continue
        bound = mx_bound(DY[:, a:b], X[:, a:b])
        assert_gemm_close(got[g], ref[g], [(0, N)], bound, what=f"wgrad[{g}]", elementwise=False)


def test_backward_gemms_exact_case(nv):
    """Small-integer MXFP8 operands: every partial sum is exact."""
    r = np.random.default_rng(950)
    counts = [40, 90]
    off, pad = _groups_from_counts(counts)
    M, N, K, G = 130, 256, 128, 2
    dy = r.integers(-4, 5, (M, N)).astype(np.float32)
    wT = r.integers(-4, 5, (K, G * N)).astype(np.float32)
    dq, de = _mx(dy)
    wq, we = _mx(wT)
    dx = nv.moe_bwd_dgrad(to_dev(dq), to_dev(de), to_dev(w8_blocked(wq, G)),
                          to_dev(w8_blocked(we, G)), to_dev(off), N, K)
    _sync()
    assert np.array_equal(from_dev(dx), GM.dgrad_grouped(dq, de, wq, we, off, N, accum="fp64").astype(np.float32))
    P = int(pad[-1])
    x = r.integers(-4, 5, (M, K)).astype(np.float32)
    dyq, dye = MX.quantize_colwise_grouped(dy, off, pad, P)
    xq, xe = MX.quantize_colwise_grouped(x, off, pad, P)
    dw = nv.moe_bwd_wgrad(to_dev(dyq), to_dev(dye), to_dev(xq), to_dev(xe), to_dev(pad), N, K)
    _sync()
    assert np.array_equal(from_dev(dw), GM.wgrad_grouped(dyq, dye, xq, xe, pad, accum="fp64").astype(np.float32))


# ------------------------------------------------------------------ launch-configuration determinism

def test_forward_and_dgrad_bits_independent_of_launch_mode(nv):
    """The same inputs in a buffer just past the routed rows (one workgroup
    per tile) and in a capacity-sized buffer (a persistent grid, one
    workgroup per compute unit looping over the tiles) give the same bits:
    each output element is accumulated by one tile in the same order in both
    launch modes. Groups: whole 256-row tiles, a 200-row partial tile and a
    4-row tail."""
    import torch
    counts, K, N = [512, 200, 260, 768], 1024, 512
    ac, asc, ao, wc, ws, wo, off = _fwd_counts_case(990, counts, K, N)
    M = int(off[-1])
    outs = []
    for cap in (M + 40, 70000):              # tile bound below / above twice the compute units
        dac = torch.zeros((cap, K // 2), dtype=torch.uint8, device="cuda")
        dac[:M] = to_dev(ac)
        das = torch.zeros((cap, K // 16), dtype=torch.uint8, device="cuda")
        das[:M] = to_dev(asc)
        dao = torch.zeros((cap,), dtype=torch.float32, device="cuda")
        dao[:M] = to_dev(ao)
        y = nv.moe_fwd_grouped_gemm(dac, das, dao, to_dev(wc), to_dev(ws), to_dev(wo), to_dev(off))
        yb = nv.moe_fwd_grouped_gemm(dac, das, dao, to_dev(wc), to_dev(ws), to_dev(wo), to_dev(off),
                                     out_dtype=torch.bfloat16)
        _sync()
        outs.append((from_dev(y)[:M], from_dev(yb)[:M]))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[1][1])
    # dgrad over the same groups: contraction N = 512, output K = 1024
    G = len(counts)
    dy = gen.normal(991, 3, (M, N), std=1e-3)
    wT = gen.normal(992, 1, (K, G * N), std=0.02)
    dq, de = _mx(dy)
    wq, we = _mx(wT)
    w8, e8 = to_dev(w8_blocked(wq, G)), to_dev(w8_blocked(we, G))
    dxs = []
    for cap in (M + 33, 70000):
        ddq = torch.zeros((cap, N), dtype=torch.uint8, device="cuda")
        ddq[:M] = to_dev(dq)
        dde = torch.zeros((cap, N // 32), dtype=torch.uint8, device="cuda")
        dde[:M] = to_dev(de)
        dx = nv.moe_bwd_dgrad(ddq, dde, w8, e8, to_dev(off), N, K)
        _sync()
        dxs.append(from_dev(dx)[:M])
    assert np.array_equal(dxs[0].view(np.uint32), dxs[1].view(np.uint32))
