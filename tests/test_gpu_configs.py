"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (ExpertLayerStep / the same entry points and shapes).

Every output is compared whole. At the expert-share and streaming sizes the
oracle runs in independent chunks on a thread pool (tests/oracle_chunks.py):
row chunks of the per-token quantizer, one expert at a time for the
per-expert quantizer and the forward GEMMs, output-row chunks of the SR
re-quantization of a transpose. Oracle inputs are the workload's own arrays
and the oracle's own results, never the GPU's.
"""

import numpy as np
import pytest

import oracle_chunks as OC
from helpers import (assert_gemm_close, ensure_built, from_dev, sr_mean_sd, to_dev, w8_tokenwise,
                     worst_elementwise)
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
    assert np.array_equal(w8_tokenwise(h(L.wT[0]), E), wq8)
    assert np.array_equal(w8_tokenwise(h(L.wT[1]), E), we8)
    dq, de = MX.quantize_rowwise(dy[:M])
    assert np.array_equal(h(L.dy8[0])[:M], dq) and np.array_equal(h(L.dy8[1])[:M], de)
    dtq, dte = MX.quantize_colwise_grouped(dy[:M], off, pad, P)
    assert np.array_equal(h(L.dyT[0])[:, :pt], dtq[:, :pt])
    assert np.array_equal(h(L.dyT[1])[:, :pt // 32], dte[:, :pt // 32])
    dx_ref = GM.dgrad_grouped(dq, de, wq8, we8, off, N)
    assert_gemm_close(h(L.dx)[:M], dx_ref.astype(np.float64), groups, what="dgrad",
                      elementwise=False)
    # (reported, not asserted: the block-scaled MFMA's in-block alignment)
    print(f"dgrad worst elementwise relative error (|ref| >= 1e-2 max): "
          f"{worst_elementwise(h(L.dx)[:M], dx_ref.astype(np.float64), groups):.3e}")
    dw_ref = GM.wgrad_grouped(dtq[:, :pt], dte[:, :pt // 32], xq8[:, :pt], xe8[:, :pt // 32], pad)
    dw = h(L.dw)
    for g in range(E):
        if pad[g + 1] > pad[g]:
            assert_gemm_close(dw[g], dw_ref[g].astype(np.float64), [(0, N)], what=f"wgrad[{g}]",
                              elementwise=False)
    print("wgrad worst elementwise relative error (|ref| >= 1e-2 max): %.3e" % max(
        worst_elementwise(dw[g], dw_ref[g].astype(np.float64), [(0, N)])
        for g in range(E) if pad[g + 1] > pad[g]))
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
    sr_w = MX.dequantize(w8_tokenwise(from_dev(L.wT[0]), E), w8_tokenwise(from_dev(L.wT[1]), E))
    e_x = from_dev(L.xT[1])[:, :pt // 32]
    e_w = w8_tokenwise(from_dev(L.wT[1]), E)
    total = 0
    for v, sr, e in ((v_x, sr_x, e_x), (v_w, sr_w, e_w)):
        bias = (sr - v).mean()
        assert abs(bias) <= 4 * sr_mean_sd(v, e) + 1e-30
        total += v.size
    assert total >= 10_000_000


def _eq(got, ref, what):
    """Bytes equal (float32 compared by bit pattern); names the first mismatch."""
    g = _bits(got) if ref.dtype == np.float32 else np.asarray(got)
    r = _bits(ref) if ref.dtype == np.float32 else ref
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    bad = np.flatnonzero((g != r).reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat index {bad[0]}"


@pytest.fixture(scope="module")
def expert_share(torch_nv):
    """32768 tokens top-8 Zipf(1.1) over 384 experts, experts 144..191 local,
    d_model 4096, FFN 4096 -> 1536 -> 4096: the GPU's quantizers, permutation
    and both forward GEMMs (float32 output), and the oracle's whole results."""
    torch, nv = torch_nv
    w = gen.expert_share()
    T, K, F_, E = w["T"], w["K"], w["N"], w["E"]
    print(f"[expert share] T={T} K={K} F={F_} E={E}", flush=True)
    d = {}
    x_d = to_dev(w["x"])
    d["xq"] = nv.nvfp4_quantize(x_d)
    d["w1q"] = nv.nvfp4_quantize(to_dev(w["w1"]), rows_per_group=F_)
    d["w2q"] = nv.nvfp4_quantize(to_dev(w["w2"]), rows_per_group=K)
    perm = nv.moe_permute(to_dev(w["topk"]), w["e0"], E, *d["xq"])
    torch.cuda.synchronize()
    M = int(perm["offsets"][-1].item())
    hid = gen.expert_share_hidden(M, F_)            # stand-in for act(Y1), bf16 [M, F]
    d["hq"] = nv.nvfp4_quantize(to_dev(hid))
    y1 = nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"], *d["w1q"],
                                 perm["offsets"], out_dtype=torch.float32)
    y2 = nv.moe_fwd_grouped_gemm(*d["hq"], *d["w2q"], perm["offsets"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    h = lambda q: tuple(from_dev(t) for t in q)
    gpu = {"xq": h(d["xq"]), "w1q": h(d["w1q"]), "w2q": h(d["w2q"]), "hq": h(d["hq"]),
           "perm": {kk: from_dev(v) for kk, v in perm.items()},
           "y1": from_dev(y1[:M]), "y2": from_dev(y2)}
    del d, perm, y1, y2, x_d
    torch.cuda.empty_cache()
    ref = {"xq": OC.quantize_rows(w["x"]), "w1q": OC.quantize_groups(w["w1"], F_),
           "w2q": OC.quantize_groups(w["w2"], K), "hq": OC.quantize_rows(hid)}
    ref["perm"] = PM.permute(w["topk"], w["e0"], E)
    ref["gath"] = PM.gather_rows(ref["perm"][2], *ref["xq"])
    return w, M, gpu, ref


def test_expert_share_quantizers_and_permute_whole(expert_share):
    """Per-token NVFP4 of X [32768, 4096] and of H [M, 1536], per-expert NVFP4
    of W1 [48 x 1536, 4096] and W2 [48 x 4096, 1536], the permutation and the
    gathered NVFP4 rows: every byte."""
    w, M, gpu, ref = expert_share
    for name in ("xq", "w1q", "w2q", "hq"):
        for i, part in enumerate(("codes", "scales", "outer")):
            _eq(gpu[name][i], ref[name][i], f"{name} {part}")
    off, pad, rt, rs = ref["perm"]
    p = gpu["perm"]
    assert M == int(off[-1]) and 0.10 * w["T"] * 8 < M < 0.14 * w["T"] * 8
    _eq(p["offsets"], off, "offsets")
    _eq(p["padded_offsets"], pad, "padded offsets")
    _eq(p["row_token"][:M], rt, "row_token")
    _eq(p["row_slot"][:M], rs, "row_slot")
    for i, part in enumerate(("codes", "scales", "outer")):
        _eq(p[part][:M], ref["gath"][i], f"gathered {part}")


def test_expert_share_forward_gemms_whole(expert_share):
    """Both forward grouped GEMMs (4096 -> 1536 on the gathered X rows,
    1536 -> 4096 on H) in float32 output on every routed row, against the
    oracle's float32 GEMM on its own quantized operands: per expert
    max|y - ref| <= 1e-3 max|ref|, and elementwise 1e-3 where |ref| >= 1e-2
    of the expert's largest."""
    w, M, gpu, ref = expert_share
    K, F_ = w["K"], w["N"]
    off = ref["perm"][0]
    groups = [(int(off[g]), int(off[g + 1])) for g in range(w["E"])]
    y1_ref = OC.fwd_grouped(ref["gath"], ref["w1q"], off, F_)
    assert_gemm_close(gpu["y1"], y1_ref.astype(np.float64), groups, what="GEMM1 4096->1536")
    del y1_ref
    y2_ref = OC.fwd_grouped(tuple(a[:M] for a in ref["hq"]), ref["w2q"], off, K)
    assert_gemm_close(gpu["y2"], y2_ref.astype(np.float64), groups, what="GEMM2 1536->4096")


def test_decode_workload(torch_nv):
    """512 tokens top-8 uniform over 384 experts, 48 local (~10 rows/expert),
    d_model 4096, FFN 1536, pre-quantized NVFP4 weights: both forward GEMMs
    (4096 -> 1536 and 1536 -> 4096) compared whole in float32 output."""
    torch, nv = torch_nv
    w = gen.decode()
    K, F_, E = w["K"], w["N"], w["E"]
    xq = nv.nvfp4_quantize(to_dev(w["x"]))
    w1q = nv.nvfp4_quantize(to_dev(w["w1"]), rows_per_group=F_)
    w2q = nv.nvfp4_quantize(to_dev(w["w2"]), rows_per_group=K)
    perm = nv.moe_permute(to_dev(w["topk"]), w["e0"], E, *xq)
    torch.cuda.synchronize()
    M = int(perm["offsets"][-1].item())
    hid = gen.expert_share_hidden(M, F_, cfg=5)
    hq = nv.nvfp4_quantize(to_dev(hid))
    y1 = nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"], *w1q, perm["offsets"])
    y2 = nv.moe_fwd_grouped_gemm(*hq, *w2q, perm["offsets"])
    torch.cuda.synchronize()
    off, pad, rt, rs = PM.permute(w["topk"], w["e0"], E)
    assert M == int(off[-1])
    xr = Q.quantize(w["x"])
    w1r = OC.quantize_groups(w["w1"], F_)
    w2r = OC.quantize_groups(w["w2"], K)
    hr = Q.quantize(hid)
    for name, got, ref in (("w1q", w1q, w1r), ("w2q", w2q, w2r), ("hq", hq, hr)):
        for i in range(3):
            _eq(from_dev(got[i]), ref[i], f"decode {name}[{i}]")
    groups = [(int(off[g]), int(off[g + 1])) for g in range(E)]
    ref1 = OC.fwd_grouped(PM.gather_rows(rt, *xr), w1r, off, F_, accum="fp64")
    assert_gemm_close(from_dev(y1)[:M], ref1, groups, what="decode GEMM1 4096->1536")
    ref2 = OC.fwd_grouped(hr, w2r, off, K, accum="fp64")
    assert_gemm_close(from_dev(y2)[:M], ref2, groups, what="decode GEMM2 1536->4096")


@pytest.fixture(scope="module")
def streaming(torch_nv):
    """1 GiB bf16 [262144 x 2048] ~ N(0, 1): per-token NVFP4 quantize, then
    the SR re-quantization of its transpose (one segment, P = 262144)."""
    torch, nv = torch_nv
    rows, cols = 262144, 2048
    x = gen.streaming(rows, cols)
    print(f"[streaming] {rows} x {cols}", flush=True)
    xd = to_dev(x)
    q = nv.nvfp4_quantize(xd)
    off = np.array([0, rows], np.int64)
    seed, tag = gen.philox_seed(5), 2
    o8, e8 = nv.mxfp8_requant_sr(*q, to_dev(off), to_dev(off), rows, seed, tag)
    torch.cuda.synchronize()
    gq = tuple(from_dev(t) for t in q)
    g8 = (from_dev(o8), from_dev(e8))
    del xd, q, o8, e8
    torch.cuda.empty_cache()
    return x, off, seed, tag, gq, g8, OC.quantize_rows(x)


def test_streaming_quantize_whole(streaming):
    """Every code, block scale and outer scale of the 1 GiB per-token quantize."""
    x, off, seed, tag, gq, g8, ref = streaming
    for i, part in enumerate(("codes", "scales", "outer")):
        _eq(gq[i], ref[i], f"streaming {part}")


def test_streaming_requant_whole(streaming):
    """Every E4M3 byte and E8M0 exponent of the SR re-quantization of the
    transpose [2048, 262144], from the oracle's own quantization of X."""
    x, off, seed, tag, gq, g8, q = streaming
    rows = x.shape[0]
    r8, re = OC.requant_cols(q, off, off, rows, seed, tag)
    _eq(g8[0], r8, "streaming requant E4M3")
    _eq(g8[1], re, "streaming requant E8M0")
