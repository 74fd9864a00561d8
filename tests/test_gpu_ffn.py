"""GPU parity of the expert FFN around the layer: the inverse permutation, the
weighted combine and its backward, the per-token re-quantization of the
intermediate, and a whole forward + backward step checked stage by stage.

Each stage's oracle input is the GPU's own output of the stages before it, so
every comparison isolates one call. Bit-exact: codes, scales, outer-scale
bits, indices, MXFP8 bytes, dY2 (a float32 product rounded once to bfloat16,
the same operations on both sides). Floating-point sums: the combine within
(k + 1) * 2^-24 * sum|g y| plus half a bfloat16 unit of the result; dgate
within the float32 bound of an N-term dot product; GEMMs the 1e-3 normwise
contract per group plus half a bfloat16 unit when stored in bfloat16.
"""

import numpy as np
import pytest

from helpers import ensure_built, from_dev, to_dev, w8_tokenwise
from oracle import ffn as FF
from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
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


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return Q._as_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _check_sum(got, ref, absmag, terms, bf16_out, what):
    """|got - ref| <= (terms + 1) 2^-24 absmag (+ 2^-8 |ref| if stored bf16)."""
    got = _f64(got)
    bound = (terms + 1) * 2.0 ** -24 * absmag + (2.0 ** -8 * np.abs(ref) if bf16_out else 0.0)
    bad = np.abs(got - ref) > bound + 1e-38
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound, worst {np.abs(got - ref).max():.3e}"


def _check_gemm(got, ref, off, bf16_out, what, tol=1e-3):
    """Per group: |got - ref| <= tol * max|ref| (+ 2^-8 |ref| if stored bf16)."""
    got = _f64(got)
    for g in range(len(off) - 1):
        a, b = int(off[g]), int(off[g + 1])
        if b <= a:
            continue
        r = ref[a:b]
        bound = tol * np.abs(r).max() + (2.0 ** -8 * np.abs(r) if bf16_out else 0.0)
        d = np.abs(got[a:b] - r)
        assert (d <= bound + 1e-38).all(), f"{what}: group {g} worst {d.max():.3e}"


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,k,N,n_exp,e0,nl,ydt,odt,gated", [
    (1000, 2, 1024, 8, 0, 8, "bf16", "bf16", True),     # all local, the small-MoE shape
    (777, 8, 256, 64, 16, 12, "bf16", "f32", True),     # most pairs not local
    (300, 3, 200, 9, 2, 5, "f32", "bf16", True),        # odd k, N not a multiple of 64
    (129, 10, 64, 16, 0, 16, "f32", "f32", False),      # k > 8 (two rounds), un-permute form
    (5, 1, 8, 4, 0, 2, "bf16", "bf16", True),           # one chunk per token
])
def test_moe_combine(nv, T, k, N, n_exp, e0, nl, ydt, odt, gated):
    import torch
    topk = gen.route_uniform(301, T, n_exp, k)
    pr = FF.pair_rows(topk, e0, nl)
    cap = T * k
    y = gen.normal(302, 4, (cap, N))
    if ydt == "bf16":
        y = gen.to_bf16_bits(y)
    gate = gen.gates(303, T, k) if gated else None
    out = nv.moe_combine(to_dev(y), to_dev(pr), None if gate is None else to_dev(gate),
                         out_dtype=torch.bfloat16 if odt == "bf16" else torch.float32)
    _sync()
    ref = FF.combine(y, pr, gate)
    absmag = FF.combine(np.abs(_f64(y)), pr, None if gate is None else np.abs(gate))
    _check_sum(from_dev(out), ref, absmag, k, odt == "bf16", "combine")


def test_moe_combine_no_local_pairs(nv):
    import torch
    T, k, N = 64, 2, 128
    pr = np.full((T, k), -1, np.int32)
    y = torch.ones((4, N), dtype=torch.bfloat16, device="cuda")
    out = nv.moe_combine(y, to_dev(pr), to_dev(gen.gates(304, T, k)))
    _sync()
    assert np.all(_f64(from_dev(out)) == 0)


@pytest.mark.parametrize("T,k,N,n_exp,e0,nl,ddt,with_y,dydt", [
    (1000, 2, 1024, 8, 0, 8, "bf16", True, "bf16"),
    (600, 8, 256, 384, 144, 48, "bf16", True, "bf16"),
    (300, 3, 520, 9, 2, 5, "f32", True, "f32"),
    (200, 2, 64, 4, 0, 4, "bf16", False, "bf16"),
])
def test_moe_combine_bwd(nv, T, k, N, n_exp, e0, nl, ddt, with_y, dydt):
    import torch
    topk = (gen.route_zipf(305, T, k=k, n_experts=n_exp) if n_exp == 384
            else gen.route_uniform(305, T, n_exp, k))
    off, _, rt, rs = PM.permute(topk, e0, nl)
    M = int(off[-1])
    cap = T * k
    dout = gen.normal(306, 3, (T, N), std=1e-3)
    if ddt == "bf16":
        dout = gen.to_bf16_bits(dout)
    y = gen.to_bf16_bits(gen.normal(307, 4, (cap, N))) if with_y else None
    gate = gen.gates(308, T, k)
    rt_d = torch.zeros(cap, dtype=torch.int32, device="cuda")
    rs_d = torch.zeros(cap, dtype=torch.int32, device="cuda")
    rt_d[:M] = to_dev(rt)
    rs_d[:M] = to_dev(rs)
    sentinel = -7.0
    dgate = torch.full((T, k), sentinel, dtype=torch.float32, device="cuda")
    dy, dg = nv.moe_combine_bwd(to_dev(dout), rt_d, rs_d, to_dev(off), k, gate=to_dev(gate),
                                y=None if y is None else to_dev(y), dgate=dgate if with_y else None,
                                dy_dtype=torch.bfloat16 if dydt == "bf16" else torch.float32)
    _sync()
    dy_ref, dg_ref = FF.combine_bwd(dout, rt, rs, M, gate, y)
    got = from_dev(dy)[:M]
    if dydt == "bf16":
        assert np.array_equal(got, FF._bf16(dy_ref))
    else:
        assert np.array_equal(_bits(got), _bits(dy_ref))
    if with_y:
        g = from_dev(dg)
        local = ~np.isnan(dg_ref)
        assert np.all(g[~local] == sentinel)
        d64 = _f64(dout)
        mag = np.zeros_like(dg_ref)
        mag[rt, rs] = np.sum(np.abs(d64[rt]) * np.abs(_f64(y)[:M]), axis=1)
        bad = np.abs(g[local] - dg_ref[local]) > (N + 1) * 2.0 ** -24 * mag[local] + 1e-38
        assert not bad.any()


# ------------------------------------------------------- live-row quantize

@pytest.mark.parametrize("M,cap,cols", [(700, 1000, 384), (0, 64, 256), (64, 64, 2048),
                                        (1, 4000, 1536)])
def test_nvfp4_quantize_live(nv, M, cap, cols):
    import torch
    x = gen.to_bf16_bits(gen.normal(309, 4, (cap, cols)))
    gen_off = to_dev(np.array([0, M], np.int64))
    codes = torch.full((cap, cols // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((cap, cols // 16), 0xCD, dtype=torch.uint8, device="cuda")
    outer = torch.full((cap,), -3.0, dtype=torch.float32, device="cuda")
    nv.nvfp4_quantize_live(to_dev(x), gen_off, codes, scales, outer)
    _sync()
    c, s, o = from_dev(codes), from_dev(scales), from_dev(outer)
    if M:
        rc, rsc, ro = Q.quantize(x[:M])
        assert np.array_equal(c[:M], rc)
        assert np.array_equal(s[:M], rsc)
        assert np.array_equal(_bits(o[:M]), _bits(ro))
    assert np.all(c[M:] == 0xAB) and np.all(s[M:] == 0xCD) and np.all(o[M:] == -3.0)


def test_permute_pair_row(nv):
    topk = gen.route_zipf(310, 2000, k=8, n_experts=384)
    x = gen.to_bf16_bits(gen.normal(310, 0, (2000, 256)))
    xq = Q.quantize(x)
    o = nv.moe_permute(to_dev(topk), 144, 48, *(to_dev(a) for a in xq))
    _sync()
    assert np.array_equal(from_dev(o["pair_row"]), FF.pair_rows(topk, 144, 48))


# ------------------------------------------------------------- whole step

@pytest.mark.parametrize("case", ["uniform", "zipf"])
def test_expert_ffn_step(nv, case):
    import torch
    from precision_moe_numerics_nvfp4_amd.layer import ExpertFFNStep
    if case == "uniform":
        c = gen.ffn_case(311, T=300, K=256, F=384, E=4, k=2)
        e0, E = 0, 4
    else:
        c = gen.ffn_case(312, T=400, K=256, F=384, E=6, k=8, routing="zipf", n_experts=384,
                         e0=144)
        e0, E = 144, 6
    T, K, F, k = c["T"], c["K"], c["F"], c["k"]
    seed = gen.philox_seed(c["cfg"])
    L = ExpertFFNStep(T, K, F, E, k, e0=e0, seed=seed)
    w1 = to_dev(c["w1"].reshape(E * F, K))
    w2 = to_dev(c["w2"].reshape(E * K, F))
    gate = to_dev(c["gate"])
    L.step(to_dev(c["x"]), w1, w2, to_dev(c["topk"]), gate, to_dev(c["dout"]))
    _sync()
    p = {kk: from_dev(v) for kk, v in L.perm.items()}
    # forward: quantizers and permutation bit-exact
    for got, ref in zip(L.xq, Q.quantize(c["x"])):
        assert np.array_equal(from_dev(got), ref)
    w1q = Q.quantize(c["w1"].reshape(E * F, K), rows_per_group=F)
    w2q = Q.quantize(c["w2"].reshape(E * K, F), rows_per_group=K)
    for got, ref in zip(L.w1q + L.w2q, w1q + w2q):
        assert np.array_equal(from_dev(got), ref)
    off, poff, rt, rs = PM.permute(c["topk"], e0, E)
    M = int(off[-1])
    assert np.array_equal(p["offsets"], off) and np.array_equal(p["padded_offsets"], poff)
    assert np.array_equal(p["row_token"][:M], rt) and np.array_equal(p["row_slot"][:M], rs)
    assert np.array_equal(p["pair_row"], FF.pair_rows(c["topk"], e0, E))
    xp = tuple(a[:M] for a in (p["codes"], p["scales"], p["outer"]))
    # up-projection, intermediate re-quantization, down-projection, combine
    h = from_dev(L.h)[:M]
    _check_gemm(h, GM.fwd_grouped(*xp, *w1q, off, F, accum="fp64"), off, True, "H")
    hq = tuple(from_dev(a)[:M] for a in L.hq)
    for got, ref in zip(hq, Q.quantize(h)):
        assert np.array_equal(got, ref)
    y2 = from_dev(L.y2)[:M]
    _check_gemm(y2, GM.fwd_grouped(*hq, *w2q, off, K, accum="fp64"), off, True, "Y2")
    pr = p["pair_row"]
    y2full = np.zeros((T * k, K), np.uint16)
    y2full[:M] = y2
    absmag = FF.combine(np.abs(_f64(y2full)), pr, c["gate"])
    _check_sum(from_dev(L.out), FF.combine(y2full, pr, c["gate"]), absmag, k, True, "out")
    # backward of the combine
    dy2_ref, dg_ref = FF.combine_bwd(c["dout"], rt, rs, M, c["gate"], y2)
    dy2 = from_dev(L.dy2)[:M]
    assert np.array_equal(dy2, FF._bf16(dy2_ref))
    local = ~np.isnan(dg_ref)
    dg = from_dev(L.dgate)
    mag = np.zeros_like(dg_ref)
    mag[rt, rs] = np.sum(np.abs(_f64(c["dout"])[rt]) * np.abs(_f64(y2)), axis=1)
    assert np.all(np.abs(dg[local] - dg_ref[local]) <= (K + 1) * 2.0 ** -24 * mag[local] + 1e-38)
    # down-projection backward
    P = L.P
    r8 = MX.quantize_rowwise(dy2)
    cT = MX.quantize_colwise_grouped(dy2, off, poff, P)
    assert np.array_equal(from_dev(L.dy2_8[0])[:M], r8[0])
    assert np.array_equal(from_dev(L.dy2_8[1])[:M], r8[1])
    pt = int(poff[-1])                   # columns past the padded total are not written
    colT = lambda pair: (from_dev(pair[0])[:, :pt], from_dev(pair[1])[:, :pt // 32])
    same = lambda a, b: np.array_equal(a[0], b[0][:, :pt]) and np.array_equal(a[1], b[1][:, :pt // 32])
    assert same(colT(L.dy2T), cT)
    hT = MX.requant_sr(*hq, off, poff, P, seed, FF.TAG_H)
    woff2 = np.arange(E + 1, dtype=np.int64) * K
    w2T = MX.requant_sr(*w2q, woff2, woff2, E * K, seed, FF.TAG_W2, rows_per_group=K)
    assert same(colT(L.hT), hT)
    for got, ref in zip(L.w2T, w2T):
        assert np.array_equal(w8_tokenwise(from_dev(got), E), ref)
    dh = from_dev(L.dh)[:M]
    _check_gemm(dh, GM.dgrad_grouped(*r8, *w2T, off, K, accum="fp64"), off, True, "dH")
    dw2_ref = GM.wgrad_grouped(*cT, *hT, poff, accum="fp64")
    dw2 = from_dev(L.dw2)
    for g in range(E):
        m = np.abs(dw2_ref[g]).max()
        assert np.abs(dw2[g] - dw2_ref[g]).max() <= 1e-3 * m + 1e-38, f"dW2 group {g}"
    # up-projection backward
    r8 = MX.quantize_rowwise(dh)
    cT = MX.quantize_colwise_grouped(dh, off, poff, P)
    assert np.array_equal(from_dev(L.dh8[0])[:M], r8[0])
    assert same(colT(L.dhT), cT)
    xT = MX.requant_sr(*xp, off, poff, P, seed, FF.TAG_X)
    woff1 = np.arange(E + 1, dtype=np.int64) * F
    w1T = MX.requant_sr(*w1q, woff1, woff1, E * F, seed, FF.TAG_W1, rows_per_group=F)
    assert same(colT(L.xT), xT)
    for got, ref in zip(L.w1T, w1T):
        assert np.array_equal(w8_tokenwise(from_dev(got), E), ref)
    dxp = from_dev(L.dxp)[:M]
    _check_gemm(dxp, GM.dgrad_grouped(*r8, *w1T, off, F, accum="fp64"), off, True, "dX_perm")
    dw1_ref = GM.wgrad_grouped(*cT, *xT, poff, accum="fp64")
    dw1 = from_dev(L.dw1)
    for g in range(E):
        m = np.abs(dw1_ref[g]).max()
        assert np.abs(dw1[g] - dw1_ref[g]).max() <= 1e-3 * m + 1e-38, f"dW1 group {g}"
    dxpfull = np.zeros((T * k, K), np.uint16)
    dxpfull[:M] = dxp
    absmag = FF.combine(np.abs(_f64(dxpfull)), pr)
    _check_sum(from_dev(L.dx), FF.combine(dxpfull, pr), absmag, k, True, "dX")
