"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (ExpertLayerStep / the same entry points and shapes).

Where the oracle can run the whole workload in seconds it does (single
expert; small MoE layer forward and backward; decode); elsewhere it computes
sampled outputs one by one: sampled token rows of the per-token quantizer,
sampled experts of the per-expert quantizer, sampled GEMM rows, sampled
output rows of the streaming re-quantization.
"""

import numpy as np
import pytest

from helpers import assert_gemm_close, ensure_built, from_dev, sr_mean_sd, to_dev
from oracle import formats as F
from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
from oracle import permute as PM
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_nv():
    ensure_built()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_moe_numerics_nvfp4_amd as nv
    return torch, nv


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _layer_run(torch, w, dy, x_dtype):
    from precision_moe_numerics_nvfp4_amd.layer import ExpertLayerStep
    L = ExpertLayerStep(w["T"], w["K"], w["N"], w["E"], w["k"], e0=w["e0"], x_dtype=x_dtype)
    L.step(to_dev(w["x"]), to_dev(w["w"]), to_dev(w["topk"]), to_dev(dy))
    torch.cuda.synchronize()
    return L


def _check_full_layer(L, w, dy, fwd_exact_rows=None):
    """Every stage of one layer step against the oracle on the whole workload."""
    h = from_dev
    N, E = w["N"], w["E"]
    xc, xs, xo = Q.quantize(w["x"])
    wc, ws, wo = Q.quantize(w["w"], rows_per_group=N)
    for got, ref in zip(L.xq, (xc, xs, xo)):
        assert np.array_equal(_bits(h(got)) if ref.dtype == np.float32 else h(got),
                              _bits(ref) if ref.dtype == np.float32 else ref)
    for got, ref in zip(L.wq, (wc, ws, wo)):
        assert np.array_equal(_bits(h(got)) if ref.dtype == np.float32 else h(got),
                              _bits(ref) if ref.dtype == np.float32 else ref)
    off, pad, rt, rs = PM.permute(w["topk"], w["e0"], E)
    M = int(off[-1])
    assert np.array_equal(h(L.perm["offsets"]), off)
    assert np.array_equal(h(L.perm["padded_offsets"]), pad)
    assert np.array_equal(h(L.perm["row_token"])[:M], rt)
    assert np.array_equal(h(L.perm["row_slot"])[:M], rs)
    ac, asc, ao = PM.gather_rows(rt, xc, xs, xo)
    assert np.array_equal(h(L.perm["codes"])[:M], ac)
    groups = [(off[g], off[g + 1]) for g in range(E)]
    y_ref = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, N)          # float32 accumulation
    assert_gemm_close(h(L.y)[:M], y_ref.astype(np.float64), groups, what="fwd")
    # backward
    P = L.P
    pt = int(pad[-1])
    xq8, xe8 = MX.requant_sr(ac, asc, ao, off, pad, P, L.seed, 0)
    assert np.array_equal(h(L.xT[0])[:, :pt], xq8[:, :pt])
    assert np.array_equal(h(L.xT[1])[:, :pt // 32], xe8[:, :pt // 32])
    woff = np.arange(E + 1) * N
    wq8, we8 = MX.requant_sr(wc, ws, wo, woff, woff, E * N, L.seed, 1, rows_per_group=N)
    assert np.array_equal(h(L.wT[0]), wq8) and np.array_equal(h(L.wT[1]), we8)
    dq, de = MX.quantize_rowwise(dy[:M])
    assert np.array_equal(h(L.dy8[0])[:M], dq) and np.array_equal(h(L.dy8[1])[:M], de)
    dtq, dte = MX.quantize_colwise_grouped(dy[:M], off, pad, P)
    assert np.array_equal(h(L.dyT[0])[:, :pt], dtq[:, :pt])
    assert np.array_equal(h(L.dyT[1])[:, :pt // 32], dte[:, :pt // 32])
    dx_ref = GM.dgrad_grouped(dq, de, wq8, we8, off, N)
    assert_gemm_close(h(L.dx)[:M], dx_ref.astype(np.float64), groups, what="dgrad",
                      elementwise=False)
    dw_ref = GM.wgrad_grouped(dtq[:, :pt], dte[:, :pt // 32], xq8[:, :pt], xe8[:, :pt // 32], pad)
    dw = h(L.dw)
    for g in range(E):
        if pad[g + 1] > pad[g]:
            assert_gemm_close(dw[g], dw_ref[g].astype(np.float64), [(0, N)], what=f"wgrad[{g}]",
                              elementwise=False)
    return dict(off=off, pad=pad, xq8=xq8, xe8=xe8, wq8=wq8, we8=we8, ac=ac, asc=asc, ao=ao,
                wc=wc, ws=ws, wo=wo)


def test_single_expert_workload(torch_nv):
    """64 tokens x 256 -> 512, fp32 with 0.1% x50 outliers, one expert."""
    torch, nv = torch_nv
    w = gen.single_expert()
    L = _layer_run(torch, w, w["dy"], torch.float32)
    _check_full_layer(L, w, w["dy"])


def test_small_moe_forward_and_backward_workload(torch_nv):
    """4096 tokens, d_model 1024, 8 experts top-2, FFN 1024 -> 2048 (bf16),
    and its backward with dY ~ N(0, 1e-6); plus the SR bias check over the
    requantized activations and weights (2.5e7 elements)."""
    torch, nv = torch_nv
    w = gen.small_moe()
    dy = gen.backward_dy(w["T"] * w["k"], w["N"])
    L = _layer_run(torch, w, dy, torch.bfloat16)
    r = _check_full_layer(L, w, dy)
    # bias of the stochastic rounding on the GPU outputs: mean(SR) - mean(v)
    off, pad = r["off"], r["pad"]
    pt = int(pad[-1])
    v_x = MX.transpose_grouped(Q.dequantize(r["ac"], r["asc"], r["ao"]), off, pad, pt).astype(np.float64)
    sr_x = MX.dequantize(from_dev(L.xT[0])[:, :pt], from_dev(L.xT[1])[:, :pt // 32])
    N, E = w["N"], w["E"]
    v_w = Q.dequantize(r["wc"], r["ws"], r["wo"], rows_per_group=N).T.astype(np.float64)
    sr_w = MX.dequantize(from_dev(L.wT[0]), from_dev(L.wT[1]))
    e_x = from_dev(L.xT[1])[:, :pt // 32]
    e_w = from_dev(L.wT[1])
    total = 0
    for v, sr, e in ((v_x, sr_x, e_x), (v_w, sr_w, e_w)):
        bias = (sr - v).mean()
        assert abs(bias) <= 5 * sr_mean_sd(v, e) + 1e-30
        total += v.size
    assert total >= 10_000_000


def test_expert_share_workload_sampled(torch_nv):
    """32768 tokens top-8 Zipf(1.1) over 384 experts, experts 144..191 local,
    d_model 4096, FFN 4096 -> 1536 -> 4096; sampled rows and experts."""
    torch, nv = torch_nv
    w = gen.expert_share()
    T, K, F_, E = w["T"], w["K"], w["N"], w["E"]
    x_d = to_dev(w["x"])
    xq = nv.nvfp4_quantize(x_d)
    w1q = nv.nvfp4_quantize(to_dev(w["w1"]), rows_per_group=F_)
    w2q = nv.nvfp4_quantize(to_dev(w["w2"]), rows_per_group=K)
    perm = nv.moe_permute(to_dev(w["topk"]), w["e0"], E, *xq)
    torch.cuda.synchronize()
    r = np.random.default_rng(31)
    # per-token quantizer on sampled tokens (a row depends on nothing else)
    rows = np.sort(r.choice(T, 512, replace=False))
    rc, rs_, ro = Q.quantize(w["x"][rows])
    assert np.array_equal(from_dev(xq[0])[rows], rc) and np.array_equal(from_dev(xq[1])[rows], rs_)
    assert np.array_equal(_bits(from_dev(xq[2])[rows]), _bits(ro))
    # per-expert quantizer on sampled experts (an expert depends on nothing else)
    for g in (0, 17, 47):
        for wt, q, n_rows in ((w["w1"], w1q, F_), (w["w2"], w2q, K)):
            sl = slice(g * n_rows, (g + 1) * n_rows)
            c, s, o = Q.quantize(wt[sl], rows_per_group=n_rows)
            assert np.array_equal(from_dev(q[0][sl]), c) and np.array_equal(from_dev(q[1][sl]), s)
            assert _bits(from_dev(q[2])[g]) == _bits(o)[0]
    # permutation: full
    off, pad, rt, rs = PM.permute(w["topk"], w["e0"], E)
    M = int(off[-1])
    assert np.array_equal(from_dev(perm["offsets"]), off)
    assert np.array_equal(from_dev(perm["row_token"])[:M], rt)
    assert 0.10 * T * 8 < M < 0.14 * T * 8
    # GEMM1 (4096 -> 1536) and GEMM2 (1536 -> 4096) on sampled rows
    h = gen.expert_share_hidden(M, F_)
    hq = nv.nvfp4_quantize(to_dev(h))
    y1 = nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"], *w1q, perm["offsets"],
                                 out_dtype=torch.bfloat16)
    y2 = nv.moe_fwd_grouped_gemm(*hq, *w2q, perm["offsets"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    pc, ps, po = (from_dev(t)[:M] for t in (perm["codes"], perm["scales"], perm["outer"]))
    hc, hs, ho = (from_dev(t) for t in hq)
    y1h, y2h = from_dev(y1[:M]), from_dev(y2)
    samp = np.sort(np.concatenate([r.choice(M, 192, replace=False), off[1:-1] - 1, off[:-1]]))
    samp = np.unique(samp[(samp >= 0) & (samp < M)])
    gidx = np.searchsorted(off, samp, side="right") - 1
    w1c, w1s, w1o = (from_dev(t) for t in w1q)
    w2c, w2s, w2o = (from_dev(t) for t in w2q)
    for rows_, g in ((samp[gidx == gg], gg) for gg in np.unique(gidx)):
        o1 = np.array([0, rows_.size])
        ref1 = GM.fwd_grouped(pc[rows_], ps[rows_], po[rows_], w1c[g * F_:(g + 1) * F_],
                              w1s[g * F_:(g + 1) * F_], w1o[g:g + 1], o1, F_, accum="fp64")
        ref2 = GM.fwd_grouped(hc[rows_], hs[rows_], ho[rows_], w2c[g * K:(g + 1) * K],
                              w2s[g * K:(g + 1) * K], w2o[g:g + 1], o1, K, accum="fp64")
        for got, ref in ((y1h[rows_], ref1), (y2h[rows_], ref2)):
            gb = F.bf16_bits_to_f32(got).astype(np.float64)
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
            assert np.all(np.abs(gb - ref) <= ulp * 1.0000001)


def test_decode_workload(torch_nv):
    """512 tokens top-8 uniform over 384 experts, 48 local (~10 rows/expert),
    d_model 4096, FFN 1536, pre-quantized NVFP4 weights: full comparison."""
    torch, nv = torch_nv
    w = gen.decode()
    K, F_, E = w["K"], w["N"], w["E"]
    xq = nv.nvfp4_quantize(to_dev(w["x"]))
    w1q = nv.nvfp4_quantize(to_dev(w["w1"]), rows_per_group=F_)
    perm = nv.moe_permute(to_dev(w["topk"]), w["e0"], E, *xq)
    y = nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"], *w1q, perm["offsets"])
    torch.cuda.synchronize()
    off, pad, rt, rs = PM.permute(w["topk"], w["e0"], E)
    M = int(off[-1])
    xc, xs, xo = Q.quantize(w["x"])
    ac, asc, ao = PM.gather_rows(rt, xc, xs, xo)
    wc, ws, wo = (from_dev(t) for t in w1q)
    ref = GM.fwd_grouped(ac, asc, ao, wc, ws, wo, off, F_, accum="fp64")
    assert_gemm_close(from_dev(y)[:M], ref, [(off[g], off[g + 1]) for g in range(E)], what="decode")


def test_streaming_quantize_and_requant_sampled(torch_nv):
    """1 GiB bf16 [262144 x 2048]: per-token NVFP4 quantize (sampled rows) and
    the SR re-quantization of its transpose (sampled output rows)."""
    torch, nv = torch_nv
    rows, cols = 262144, 2048
    x = gen.streaming(rows, cols)
    xd = to_dev(x)
    q = nv.nvfp4_quantize(xd)
    off = np.array([0, rows], np.int64)
    seed, tag = gen.philox_seed(5), 2
    o8, e8 = nv.mxfp8_requant_sr(*q, to_dev(off), to_dev(off), rows, seed, tag)
    torch.cuda.synchronize()
    del xd
    r = np.random.default_rng(55)
    samp = np.sort(r.choice(rows, 1024, replace=False))
    rc, rs_, ro = Q.quantize(x[samp])
    qc, qs, qo = (from_dev(t) for t in q)
    assert np.array_equal(qc[samp], rc) and np.array_equal(qs[samp], rs_)
    assert np.array_equal(_bits(qo[samp]), _bits(ro))
    got8 = from_dev(o8)
    gote = from_dev(e8)
    for k in (0, 1, 777, 2047):
        kb = k // 16
        v = Q.dequantize(np.ascontiguousarray(qc[:, kb * 8:(kb + 1) * 8]),
                         np.ascontiguousarray(qs[:, kb:kb + 1]), qo)[:, k % 16]
        c, e = MX.quantize_sr(v[None, :], seed, tag, idx_base=k * rows)
        assert np.array_equal(got8[k], c[0]) and np.array_equal(gote[k], e[0])
