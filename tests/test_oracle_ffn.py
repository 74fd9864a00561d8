"""Pins of the oracle's expert FFN (combine, its backward, and the forward and
backward compositions), CPU only.

* pair_rows: brute-force rank counting agrees with the permutation's
  (row_token, row_slot) from the other direction.
* combine: plain Python loops on a tiny case; combine of gathered rows is the
  row scaled by the sum of its local gates (closed form).
* combine backward: the adjoint identity <combine(y, g), d> = <y, dy>, and
  dgate equals the change of <combine(y, g), d> when one gate moves by one
  (combine is linear in each gate).
* FFN forward and backward: within the quantization error of the unquantized
  float64 FFN computed with per-pair matrix-vector loops; the backward within
  MXFP8's error of the exact gradients of the forward's own quantized operands.
  Dropping the routing weights, a transposed weight or a wrong row would put
  the error near or above one.
"""

import numpy as np

from oracle import ffn as FF
from oracle import nvfp4 as Q
from oracle import permute as PM
from workloads import gen


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def test_pair_rows_inverse_of_permutation():
    for seed, T, k, n_exp, e0, nl in [(71, 50, 3, 9, 2, 4), (72, 33, 2, 5, 0, 5), (73, 8, 4, 16, 12, 4)]:
        topk = gen.route_uniform(seed, T, n_exp, k)
        pr = FF.pair_rows(topk, e0, nl)
        off, _, rt, rs = PM.permute(topk, e0, nl)
        M = int(off[-1])
        assert np.array_equal(np.sort(pr[pr >= 0]), np.arange(M))
        for r in range(M):
            assert pr[rt[r], rs[r]] == r
        for t in range(T):
            for j in range(k):
                assert (pr[t, j] >= 0) == (e0 <= topk[t, j] < e0 + nl)


def test_combine_bruteforce():
    rng = np.random.default_rng(5)
    T, k, N, M = 7, 3, 5, 12
    y = rng.standard_normal((M, N))
    pr = np.array([[0, 4, -1], [1, -1, 5], [2, 6, 8], [-1, -1, -1], [3, 7, 9], [10, -1, 11],
                   [-1, -1, -1]], dtype=np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    out = FF.combine(y, pr, gate)
    for t in range(T):
        for n in range(N):
            s = 0.0
            for j in range(k):
                if pr[t, j] >= 0:
                    s += float(gate[t, j]) * y[pr[t, j], n]
            assert abs(out[t, n] - s) <= 1e-12 * (1 + abs(s))
    assert np.all(FF.combine(y, pr)[3] == 0)


def test_combine_of_gathered_rows():
    T, k, K, n_exp = 40, 3, 24, 6
    topk = gen.route_uniform(74, T, n_exp, k)
    z = gen.normal(74, 0, (T, K)).astype(np.float64)
    gate = gen.gates(74, T, k)
    e0, nl = 1, 4
    off, _, rt, rs = PM.permute(topk, e0, nl)
    pr = FF.pair_rows(topk, e0, nl)
    y = z[rt[:int(off[-1])]]
    local = (topk >= e0) & (topk < e0 + nl)
    expect = z * np.where(local, gate.astype(np.float64), 0.0).sum(axis=1)[:, None]
    assert np.allclose(FF.combine(y, pr, gate), expect, rtol=1e-12, atol=1e-12)


def test_combine_backward_adjoint_and_gate_derivative():
    T, k, K, n_exp, e0, nl = 30, 2, 16, 5, 0, 3
    topk = gen.route_uniform(75, T, n_exp, k)
    off, _, rt, rs = PM.permute(topk, e0, nl)
    M = int(off[-1])
    pr = FF.pair_rows(topk, e0, nl)
    gate = gen.gates(75, T, k)
    y = gen.normal(75, 4, (M, K)).astype(np.float64)
    d = gen.normal(75, 3, (T, K))
    dy, dg = FF.combine_bwd(d, rt, rs, M, gate, y)
    lhs = float(np.sum(FF.combine(y, pr, gate) * d))
    rhs = float(np.sum(y * dy.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-6 * float(np.sum(np.abs(y) * np.abs(dy)))
    base = FF.combine(y, pr, gate)
    for t, j in [(0, 0), (3, 1), (T - 1, 0)]:
        if pr[t, j] < 0:
            assert np.isnan(dg[t, j])
            continue
        g2 = gate.astype(np.float64).copy()
        g2[t, j] += 1.0
        delta = float(np.sum((FF.combine(y, pr, g2) - base) * d))
        assert abs(delta - dg[t, j]) <= 1e-10 * (1 + abs(delta))


def _case():
    c = gen.ffn_case(81, T=96, K=128, F=192, E=4, k=2)
    return c, FF.ffn_forward(c["x"], c["w1"], c["w2"], c["topk"], c["gate"], 0, 4)


def _exact_ffn(c):
    """Unquantized FFN and its gradients, one (token, slot) pair at a time."""
    x = Q._as_f32(c["x"]).astype(np.float64)
    w1 = Q._as_f32(c["w1"]).astype(np.float64)
    w2 = Q._as_f32(c["w2"]).astype(np.float64)
    d = Q._as_f32(c["dout"]).astype(np.float64)
    g = c["gate"].astype(np.float64)
    topk = c["topk"]
    T, K = x.shape
    k = topk.shape[1]
    out, dx = np.zeros((T, K)), np.zeros((T, K))
    dw1, dw2, dg = np.zeros_like(w1), np.zeros_like(w2), np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = topk[t, j]
            h = w1[e] @ x[t]
            y = w2[e] @ h
            out[t] += g[t, j] * y
            dy = g[t, j] * d[t]
            dg[t, j] = d[t] @ y
            dh = w2[e].T @ dy
            dw2[e] += np.outer(dy, h)
            dx[t] += w1[e].T @ dh
            dw1[e] += np.outer(dh, x[t])
    return dict(out=out, dx=dx, dw1=dw1, dw2=dw2, dgate=dg)


def test_ffn_within_quantization_error_of_exact():
    c, fw = _case()
    bw = FF.ffn_backward(c["dout"], fw, c["gate"], gen.philox_seed(81))
    ex = _exact_ffn(c)
    # NVFP4 operands in two chained matmuls: ~0.19 measured; unrelated results are >= 1
    assert _rel(Q._as_f32(fw["out"]), ex["out"]) < 0.3
    for key in ("dw1", "dw2", "dgate"):
        assert _rel(bw[key], ex[key]) < 0.3, key
    assert _rel(Q._as_f32(bw["dx"]), ex["dx"]) < 0.3
    # the routing weights matter: the same sum without them is far off
    pr = fw["pair_row"]
    no_gate = Q._as_f32(FF._bf16(FF.combine(fw["y2"], pr).astype(np.float32)))
    assert _rel(no_gate, ex["out"]) > 0.5


def test_ffn_backward_within_mxfp8_error_of_its_operands():
    c, fw = _case()
    bw = FF.ffn_backward(c["dout"], fw, c["gate"], gen.philox_seed(81))
    off = fw["offsets"]
    M = int(off[-1])
    E, Fw, K = 4, 192, 128
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    hq = Q.dequantize(*fw["hq"]).astype(np.float64)
    xp = Q.dequantize(*fw["xp"]).astype(np.float64)
    W1 = Q.dequantize(*fw["w1q"], rows_per_group=Fw).reshape(E, Fw, K)
    W2 = Q.dequantize(*fw["w2q"], rows_per_group=K).reshape(E, K, Fw)
    dy2 = Q._as_f32(bw["dy2"]).astype(np.float64)
    dh = Q._as_f32(bw["dh"]).astype(np.float64)
    dh_e = np.stack([W2[grp[r]].T @ dy2[r] for r in range(M)])
    dxp_e = np.stack([W1[grp[r]].T @ dh[r] for r in range(M)])
    dw2_e, dw1_e = np.zeros((E, K, Fw)), np.zeros((E, Fw, K))
    for r in range(M):
        dw2_e[grp[r]] += np.outer(dy2[r], hq[r])
        dw1_e[grp[r]] += np.outer(dh[r], xp[r])
    # E4M3 elements (3 mantissa bits) on both operands: ~0.046 measured
    assert _rel(dh, dh_e) < 0.08
    assert _rel(Q._as_f32(bw["dxp"]), dxp_e) < 0.08
    assert _rel(bw["dw2"], dw2_e) < 0.08
    assert _rel(bw["dw1"], dw1_e) < 0.08
    # dY2 is the gate times the token's output gradient, rounded once to bfloat16
    rt, rs = fw["row_token"][:M], fw["row_slot"][:M]
    d = Q._as_f32(c["dout"]).astype(np.float64)
    ref = c["gate"].astype(np.float64)[rt, rs][:, None] * d[rt]
    assert np.all(np.abs(dy2 - ref) <= np.abs(ref) * 2.0 ** -8)
