"""The expert FFN around the quantized path: down-projection, per-token NVFP4
re-quantization of the intermediate activation, the weighted combine back to
token order, and the backward pass through both projections.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the expert layers' matmuls run in NVFP4 forward and MXFP8 backward
("Inkling 2 Small uses four-bit training ...", ai-primer, section "NVFP4
forward, MXFP8 backward"); every expert matmul input is NVFP4 with one outer
scale per token (activations) or per expert (weights) (same page, section
"Block scales and per-token activations"); tokens are dispatched to their
experts and the expert outputs are combined back (section "Quantized NVLink
and BBBK"; the Hadamard + S2F6 transfer format of that combine is a
communication step between GPUs and is not part of this computation).

Readings (the pages give no FFN details):
* One expert's FFN is an up-projection W1 [F, K] and a down-projection
  W2 [K, F]; the nonlinearity between them is not on the pages and is left to
  the caller, so the intermediate activation H is the up-projection's output.
* H is produced in bfloat16 and re-quantized to NVFP4 per routed row (one
  outer scale per token of that expert), like the layer's input.
* Stored precisions: H, the down-projection output Y2, dY2, dH and dX_perm are
  bfloat16 (round to nearest even from the float32 accumulator); the combine
  and the un-permute accumulate k terms in float32 in slot order and store
  bfloat16.
* combine: out[t] = sum over slots j whose expert is local of
  gate[t, j] * Y2[row(t, j)]; un-permute is the same with gate = 1.
* combine backward: dY2[r] = gate[t, j] * dOut[t] (a float32 product, stored
  bfloat16) and dgate[t, j] = sum_n dOut[t, n] * Y2[r, n].
* Each projection's backward is the layer's MXFP8 path: saved NVFP4 operands
  re-quantized with stochastic rounding (Philox tags 0 = X_perm, 1 = W1,
  3 = H, 4 = W2), the output gradient quantized RNE in both orientations,
  dgrad and wgrad in MXFP8.
"""

import numpy as np

from . import formats as F
from . import nvfp4 as Q
from . import mxfp8 as MX
from . import permute as P
from . import gemm as G

TAG_X, TAG_W1, TAG_H, TAG_W2 = 0, 1, 3, 4


def _vals(x):
    """bfloat16 bit patterns (uint16) or floats -> float64 values."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return F.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def pair_rows(topk_ids, e0, n_local):
    """Row of the permuted order holding each routed pair, -1 if its expert is
    not local: row(t, j) = offsets[e] + #{(t', j') before (t, j) in flat order
    with the same expert e}. Returns int32 [T, k]."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    counts = np.zeros(n_local, dtype=np.int64)
    flat = ids.reshape(-1)
    for f in range(flat.shape[0]):
        e = flat[f] - e0
        if 0 <= e < n_local:
            counts[e] += 1
    start = np.concatenate([[0], np.cumsum(counts)])
    seen = np.zeros(n_local, dtype=np.int64)
    out = np.full(flat.shape[0], -1, dtype=np.int32)
    for f in range(flat.shape[0]):
        e = flat[f] - e0
        if 0 <= e < n_local:
            out[f] = start[e] + seen[e]
            seen[e] += 1
    return out.reshape(T, k)


def combine(y, pair_row, gate=None):
    """out[t, :] = sum_j gate[t, j] * y[pair_row[t, j], :] over local pairs, in
    float64. y: [rows, N] float or bfloat16 bits; gate None means 1."""
    v = _vals(y)
    pr = np.asarray(pair_row, dtype=np.int64)
    T, k = pr.shape
    out = np.zeros((T, v.shape[1]), dtype=np.float64)
    for j in range(k):
        r = pr[:, j]
        m = r >= 0
        g = np.ones(T) if gate is None else np.asarray(gate, dtype=np.float64)[:, j]
        out[m] += g[m, None] * v[r[m]]
    return out


def combine_bwd(dout, row_token, row_slot, M, gate, y=None):
    """Backward of combine for the M routed rows.

    dy[r] = gate[t, j] * dout[t] as a float32 product (the value the stored
    bfloat16 is rounded from); dgate[t, j] = sum_n dout[t, n] * y[r, n] in
    float64 for local pairs (NaN elsewhere: not written). Returns (dy float32
    [M, N], dgate float64 [T, k] or None)."""
    d = Q._as_f32(dout)
    rt = np.asarray(row_token, dtype=np.int64)[:M]
    rs = np.asarray(row_slot, dtype=np.int64)[:M]
    g = np.asarray(gate, dtype=np.float32)
    dy = (g[rt, rs][:, None] * d[rt]).astype(np.float32)
    if y is None:
        return dy, None
    v = _vals(y)[:M]
    dgate = np.full(g.shape, np.nan)
    dgate[rt, rs] = np.sum(d[rt].astype(np.float64) * v, axis=1)
    return dy, dgate


def _bf16(x):
    return F.f32_to_bf16_bits_rne(np.asarray(x, dtype=np.float32))


def ffn_forward(x, w1, w2, topk_ids, gate, e0, n_local):
    """Forward of the routed expert FFN. x [T, K], w1 [E, F, K], w2 [E, K, F]
    (float or bfloat16 bits). Returns a dict of every stored intermediate."""
    w1 = np.asarray(w1)
    w2 = np.asarray(w2)
    E, Fw, K = w1.shape
    xq = Q.quantize(x)
    w1q = Q.quantize(w1.reshape(E * Fw, K), rows_per_group=Fw)
    w2q = Q.quantize(w2.reshape(E * K, Fw), rows_per_group=K)
    off, poff, rt, rs = P.permute(topk_ids, e0, n_local)
    xp = P.gather_rows(rt, *xq)
    h = _bf16(G.fwd_grouped(*xp, *w1q, off, Fw))            # [M, F] bfloat16 bits
    hq = Q.quantize(h)
    y2 = _bf16(G.fwd_grouped(*hq, *w2q, off, K))            # [M, K] bfloat16 bits
    pr = pair_rows(topk_ids, e0, n_local)
    out = _bf16(combine(y2, pr, gate).astype(np.float32))
    return dict(xq=xq, w1q=w1q, w2q=w2q, offsets=off, padded_offsets=poff, row_token=rt,
                row_slot=rs, pair_row=pr, xp=xp, h=h, hq=hq, y2=y2, out=out)


def ffn_backward(dout, fwd, gate, seed):
    """Backward of ffn_forward for the output gradient dout [T, K]. Returns a
    dict with dy2, dh, dxp (bfloat16 bits), dgate, dw2 [E, K, F], dw1 [E, F, K]
    (float32) and dx (bfloat16 bits)."""
    off, poff = fwd["offsets"], fwd["padded_offsets"]
    M = int(off[-1])
    E = off.shape[0] - 1
    Pw = max(32, int(poff[-1]))                             # padded token width
    Fw = fwd["h"].shape[1]
    K = fwd["y2"].shape[1]
    dy2f, dgate = combine_bwd(dout, fwd["row_token"], fwd["row_slot"], M, gate, fwd["y2"])
    dy2 = _bf16(dy2f)
    # down-projection: operands H (saved NVFP4 per row) and W2 (per expert)
    w_off2 = np.arange(E + 1, dtype=np.int64) * K
    hT = MX.requant_sr(*fwd["hq"], off, poff, Pw, seed, TAG_H)
    w2T = MX.requant_sr(*fwd["w2q"], w_off2, w_off2, E * K, seed, TAG_W2, rows_per_group=K)
    dy8 = MX.quantize_rowwise(dy2)
    dyT = MX.quantize_colwise_grouped(dy2, off, poff, Pw)
    dh = _bf16(G.dgrad_grouped(*dy8, *w2T, off, K))         # [M, F]
    dw2 = G.wgrad_grouped(*dyT, *hT, poff)                  # [E, K, F]
    # up-projection: operands X_perm (saved NVFP4 per row) and W1 (per expert)
    w_off1 = np.arange(E + 1, dtype=np.int64) * Fw
    xT = MX.requant_sr(*fwd["xp"], off, poff, Pw, seed, TAG_X)
    w1T = MX.requant_sr(*fwd["w1q"], w_off1, w_off1, E * Fw, seed, TAG_W1, rows_per_group=Fw)
    dh8 = MX.quantize_rowwise(dh)
    dhT = MX.quantize_colwise_grouped(dh, off, poff, Pw)
    dxp = _bf16(G.dgrad_grouped(*dh8, *w1T, off, Fw))       # [M, K]
    dw1 = G.wgrad_grouped(*dhT, *xT, poff)                  # [E, F, K]
    dx = _bf16(combine(dxp, fwd["pair_row"]).astype(np.float32))
    return dict(dy2=dy2, dgate=dgate, dh=dh, dw2=dw2, dxp=dxp, dw1=dw1, dx=dx, P=Pw)
