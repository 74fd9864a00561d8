"""Whole-tensor oracle results at the full workload sizes, computed in
independent chunks on a thread pool (numpy releases the interpreter lock in
its array loops). Each chunk is a plain call of the oracle on a slice whose
result depends on nothing outside it:

* per-row NVFP4 quantization: a row depends only on itself;
* per-group NVFP4 quantization: a group of rows (one expert) only on itself;
* the SR re-quantization of a transpose: output rows c0..c0+n depend only on
  input columns c0..c0+n, and their draws keep the absolute linear index
  c0 * P + ... of the output buffer;
* the forward grouped GEMM: a group's rows only on that group's operands.

Test infrastructure only, like the oracle it calls.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q

THREADS = max(1, min(16, os.cpu_count() or 1))


def _map(fn, items, threads=THREADS):
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def quantize_rows(x, chunk=4096):
    """Q.quantize(x) with one outer scale per row, row chunk by row chunk."""
    rows = x.shape[0]
    parts = _map(lambda r0: Q.quantize(x[r0:r0 + chunk]), range(0, rows, chunk))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def quantize_groups(w, rows_per_group):
    """Q.quantize(w, rows_per_group) one group (expert) at a time."""
    G = w.shape[0] // rows_per_group
    parts = _map(lambda g: Q.quantize(w[g * rows_per_group:(g + 1) * rows_per_group],
                                      rows_per_group=rows_per_group), range(G))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def requant_cols(q, offsets, padded_offsets, P, seed, tag, rows_per_group=None, ncols=64):
    """MX.requant_sr(*q, ...) as output-row chunks of ncols (a multiple of 32):
    returns (E4M3 [cols, P], E8M0 [cols, P/32])."""
    codes, scales, outer = q
    cols = codes.shape[1] * 2

    def one(c0):
        v = Q.dequantize(codes[:, c0 // 2:(c0 + ncols) // 2],
                         scales[:, c0 // 16:(c0 + ncols) // 16], outer,
                         rows_per_group=rows_per_group)
        t = MX.transpose_grouped(v, offsets, padded_offsets, P)
        return MX.quantize_sr(t, seed, tag, idx_base=c0 * P)

    parts = _map(one, range(0, cols, ncols))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def fwd_grouped(a, b, offsets, N, accum="fp32", threads=4):
    """GM.fwd_grouped on NVFP4 operands a = (codes, scales, outer) [M rows],
    b = (codes, scales, outer) [G*N rows, outer per group], group by group:
    returns float32 (or float64) [M, N]."""
    off = np.asarray(offsets, dtype=np.int64)
    G = off.shape[0] - 1
    M = int(off[-1])
    out = np.zeros((M, N), dtype=np.float64 if accum == "fp64" else np.float32)

    def one(g):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            return
        out[r0:r1] = GM.fwd_grouped(a[0][r0:r1], a[1][r0:r1], a[2][r0:r1],
                                    b[0][g * N:(g + 1) * N], b[1][g * N:(g + 1) * N],
                                    b[2][g:g + 1], np.array([0, r1 - r0]), N, accum=accum)

    _map(one, range(G), threads)
    return out
