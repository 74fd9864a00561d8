"""The chunked oracle driver (tests/oracle_chunks.py) gives exactly the
oracle's whole-tensor results: row chunks, expert chunks, output-row chunks
of the SR re-quantization (absolute draw indices) and per-expert GEMMs."""

import numpy as np

import oracle_chunks as OC
from oracle import gemm as GM
from oracle import mxfp8 as MX
from oracle import nvfp4 as Q
from workloads import gen


def test_quantize_chunks_equal_whole():
    x = gen.to_bf16_bits(gen.normal(901, 0, (1000, 96)))
    for a, b in zip(OC.quantize_rows(x, chunk=128), Q.quantize(x)):
        assert np.array_equal(a, b)
    w = gen.to_bf16_bits(gen.normal(901, 1, (6 * 64, 96), std=0.02))
    for a, b in zip(OC.quantize_groups(w, 64), Q.quantize(w, rows_per_group=64)):
        assert np.array_equal(a, b)


def test_requant_chunks_equal_whole():
    x = gen.to_bf16_bits(gen.normal(902, 0, (300, 128)))
    q = Q.quantize(x)
    off = np.array([0, 37, 37, 200, 300], np.int64)
    pad = MX.padded_offsets_from_offsets(off)
    P = int(pad[-1]) + 32
    whole = MX.requant_sr(*q, off, pad, P, 0x1234, 0)
    chunked = OC.requant_cols(q, off, pad, P, 0x1234, 0, ncols=32)
    assert np.array_equal(whole[0], chunked[0]) and np.array_equal(whole[1], chunked[1])
    w = gen.to_bf16_bits(gen.normal(902, 1, (4 * 64, 128), std=0.02))
    qw = Q.quantize(w, rows_per_group=64)
    woff = np.arange(5, dtype=np.int64) * 64
    whole = MX.requant_sr(*qw, woff, woff, 256, 7, 1, rows_per_group=64)
    chunked = OC.requant_cols(qw, woff, woff, 256, 7, 1, rows_per_group=64, ncols=64)
    assert np.array_equal(whole[0], chunked[0]) and np.array_equal(whole[1], chunked[1])


def test_gemm_chunks_equal_whole():
    x = gen.to_bf16_bits(gen.normal(903, 0, (90, 64)))
    w = gen.to_bf16_bits(gen.normal(903, 1, (3 * 48, 64), std=0.02))
    a = Q.quantize(x)
    b = Q.quantize(w, rows_per_group=48)
    off = np.array([0, 40, 40, 90], np.int64)
    for acc in ("fp32", "fp64"):
        whole = GM.fwd_grouped(*a, *b, off, 48, accum=acc)
        assert np.array_equal(OC.fwd_grouped(a, b, off, 48, accum=acc), whole)
