"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host before touching the GPU (CPU only: no
compute call is made)."""

import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"NVFP4MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


@pytest.fixture(scope="module")
def L():
    ensure_built()
    from precision_moe_numerics_nvfp4_amd import binding
    return binding.lib()


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"nvfp4_quantize", "mxfp8_requant_sr", "moe_fwd_grouped_gemm", "moe_bwd_dgrad",
            "moe_bwd_wgrad", "moe_permute", "mxfp8_quantize"} <= names


def test_every_declared_symbol_is_exported(L):
    from precision_moe_numerics_nvfp4_amd import binding
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in binding.SIGNATURES, f"binding lacks {name}"


def test_version_and_status_strings(L):
    from precision_moe_numerics_nvfp4_amd import binding
    assert L.nvfp4moe_abi_version() == 3
    for s, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported size or alignment"),
                    (3, "workspace too small"), (4, "HIP launch or runtime error"), (99, "unknown status")]:
        assert binding.status_string(s) == text


def test_workspace_size(L):
    assert L.nvfp4moe_permute_workspace_size(32768, 8, 48) >= 256 * 48 * 4
    assert L.nvfp4moe_permute_workspace_size(-1, 8, 48) == 0
    assert L.nvfp4moe_permute_workspace_size(10, 0, 48) == 0


EINVAL, EUNSUP, EWS = 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: calls fail first
FAKE_MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only


def test_quantize_argument_errors(L):
    q = L.nvfp4_quantize
    assert q(None, 1, 4, 64, 0, 0, FAKE, FAKE, FAKE, None) == EINVAL          # null x
    assert q(FAKE, 7, 4, 64, 0, 0, FAKE, FAKE, FAKE, None) == EINVAL          # bad dtype
    assert q(FAKE, 1, -1, 64, 0, 0, FAKE, FAKE, FAKE, None) == EINVAL         # negative rows
    assert q(FAKE, 1, 4, 64, 5, 0, FAKE, FAKE, FAKE, None) == EINVAL          # bad mode
    assert q(FAKE, 1, 4, 64, 1, 0, FAKE, FAKE, FAKE, None) == EINVAL          # group of 0 rows
    assert q(FAKE, 1, 4, 48, 0, 0, FAKE, FAKE, FAKE, None) == EUNSUP          # cols % 32
    assert q(FAKE, 1, 6, 64, 1, 4, FAKE, FAKE, FAKE, None) == EUNSUP          # rows % group
    assert q(FAKE_MIS, 1, 4, 64, 0, 0, FAKE, FAKE, FAKE, None) == EUNSUP      # alignment
    assert q(None, 1, 0, 64, 0, 0, None, None, None, None) == 0               # empty is a no-op


def test_gemm_and_requant_argument_errors(L):
    g = L.moe_fwd_grouped_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 64, 256, 256, FAKE, 0, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 200, 256, FAKE, 0, None) == EUNSUP
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 256, 256, FAKE, 3, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 256, 256, FAKE, 0, None) == 0
    r = L.mxfp8_requant_sr
    assert r(FAKE, FAKE, FAKE, 0, 0, 64, 256, FAKE, FAKE, 1, 48, 1, 0, FAKE, FAKE, None) == EUNSUP
    assert r(FAKE, FAKE, FAKE, 2, 0, 64, 256, FAKE, FAKE, 1, 64, 1, 0, FAKE, FAKE, None) == EINVAL
    assert r(FAKE, FAKE, FAKE, 0, 0, 64, 256, None, FAKE, 1, 64, 1, 0, FAKE, FAKE, None) == EINVAL
    d = L.moe_bwd_dgrad
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 100, 256, FAKE, 0, None) == EUNSUP
    w = L.moe_bwd_wgrad
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 40, 128, 128, FAKE, None) == EUNSUP
    assert w(None, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, FAKE, None) == EINVAL
    # 32-bit tile offsets and the in-kernel group ranking bound the sizes
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 16711936, 256, FAKE, 0, None) == EUNSUP
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16711936 + 32 - 16711936 % 32, 128, 128, FAKE,
             None) == EUNSUP
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 16385, 64, 128, 128, FAKE, None) == EUNSUP
    f8 = L.moe_fwd_grouped_gemm_mxfp8
    assert f8(FAKE, FAKE, FAKE, FAKE, None, 2, 64, 256, 256, FAKE, 0, None) == EINVAL   # no offsets
    assert f8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 256, 256, FAKE, 5, None) == EINVAL   # bad dtype
    assert f8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 200, 256, FAKE, 0, None) == EUNSUP   # N % 128
    assert f8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 256, 96, FAKE, 0, None) == EUNSUP    # K % 128
    assert f8(FAKE_MIS, FAKE, FAKE, FAKE, FAKE, 2, 64, 256, 256, FAKE, 0, None) == EUNSUP
    assert f8(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 256, 256, FAKE, 0, None) == 0         # nothing to do
    t16 = L.nvfp4_quantize_tile16
    assert t16(FAKE, 1, 64, 256, 0, FAKE, FAKE, FAKE, None) == EINVAL           # rows_per_group 0
    assert t16(FAKE, 1, 40, 256, 40, FAKE, FAKE, FAKE, None) == EUNSUP          # rows % 16
    assert t16(FAKE, 1, 64, 256, 24, FAKE, FAKE, FAKE, None) == EUNSUP          # group % 16
    assert t16(FAKE, 1, 64, 200, 64, FAKE, FAKE, FAKE, None) == EUNSUP          # cols % 16
    assert t16(None, 1, 64, 256, 64, FAKE, FAKE, FAKE, None) == EINVAL
    qd = L.mxfp8_quantize_dual
    assert qd(FAKE, 1, 64, 256, None, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert qd(FAKE, 1, 64, 96, FAKE, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == EUNSUP
    assert qd(FAKE, 1, 64, 256, FAKE, FAKE, 2, 100, FAKE, FAKE, FAKE, FAKE, None) == EUNSUP
    gr = L.mxfp8_gather_rows
    assert gr(None, FAKE, 2, 64, FAKE, FAKE, 10, 256, FAKE, FAKE, None) == EINVAL
    assert gr(FAKE, FAKE, 2, 64, FAKE, FAKE, 10, 48, FAKE, FAKE, None) == EUNSUP        # K % 32
    assert gr(FAKE, FAKE, 2, 64, FAKE, FAKE, -1, 256, FAKE, FAKE, None) == EINVAL
    m = L.mxfp8_quantize
    assert m(FAKE, 1, 64, 256, 9, None, None, 0, 0, FAKE, FAKE, None) == EINVAL
    assert m(FAKE, 1, 64, 48, 0, None, None, 0, 0, FAKE, FAKE, None) == EUNSUP


def test_permute_argument_errors(L):
    p = L.moe_permute
    args = lambda T, k, nl, K, ws, wsb: (FAKE, T, k, 0, nl, FAKE, FAKE, FAKE, K, FAKE, FAKE, FAKE,
                                         FAKE, None, FAKE, FAKE, FAKE, ws, wsb, None)
    need = L.nvfp4moe_permute_workspace_size(100, 2, 8)
    assert p(*args(100, 2, 8, 256, FAKE, need - 1)) == EWS
    assert p(*args(100, 2, 8, 48, FAKE, need)) == EUNSUP
    assert p(*args(100, 2, 2000, 256, FAKE, 1 << 30)) == EUNSUP
    assert p(*args(100, 0, 8, 256, FAKE, need)) == EINVAL
    assert p(*args(100, 2, 8, 256, None, need)) == EINVAL


def test_ffn_entry_argument_errors(L):
    ql = L.nvfp4_quantize_live
    assert ql(FAKE, 1, 64, 256, None, FAKE, FAKE, FAKE, None) == EINVAL            # n_live
    assert ql(FAKE, 1, 64, 48, FAKE, FAKE, FAKE, FAKE, None) == EUNSUP             # cols % 32
    assert ql(FAKE, 1, 64, 16384, FAKE, FAKE, FAKE, FAKE, None) == EUNSUP          # cols > 8192
    assert ql(FAKE, 7, 64, 256, FAKE, FAKE, FAKE, FAKE, None) == EINVAL            # dtype
    assert ql(None, 1, 0, 256, None, None, None, None, None) == 0                  # empty
    c = L.moe_combine
    assert c(FAKE, 1, 64, 32, 2, 256, None, None, FAKE, 1, None) == EINVAL         # pair_row
    assert c(FAKE, 1, 0, 32, 2, 256, FAKE, None, FAKE, 1, None) == EINVAL          # m_cap 0
    assert c(FAKE, 1, 64, 32, 2, 252, FAKE, None, FAKE, 1, None) == EUNSUP         # N % 8
    assert c(FAKE, 1, 64, 32, 65, 256, FAKE, None, FAKE, 1, None) == EUNSUP        # k > 64
    assert c(FAKE, 1, 64, 32, 0, 256, FAKE, None, FAKE, 1, None) == EINVAL         # k 0
    assert c(FAKE, 1, 64, 32, 2, 256, FAKE, None, FAKE, 5, None) == EINVAL         # out dtype
    assert c(None, 1, 0, 0, 2, 256, None, None, None, 1, None) == 0                # no tokens
    b = L.moe_combine_bwd
    assert b(FAKE, 1, 32, 2, 256, FAKE, FAKE, None, 2, 64, None, None, 0, FAKE, 1, None,
             None) == EINVAL                                                        # offsets
    assert b(FAKE, 1, 32, 2, 256, FAKE, FAKE, FAKE, 2, 64, None, FAKE, 1, FAKE, 1, None,
             None) == EINVAL                                                        # y without dgate
    assert b(FAKE, 1, 32, 2, 250, FAKE, FAKE, FAKE, 2, 64, None, None, 0, FAKE, 1, None,
             None) == EUNSUP                                                        # N % 8
    assert b(FAKE, 1, 32, 2, 256, FAKE, FAKE, FAKE, 0, 64, None, None, 0, FAKE, 1, None,
             None) == 0                                                             # no groups


def test_nvfp4_backward_entry_argument_errors(L):
    po = L.moe_padded_offsets
    assert po(FAKE, 4, 0, FAKE, None) == EINVAL                                    # align 0
    assert po(FAKE, 2000, 128, FAKE, None) == EUNSUP                               # G > 1024
    assert po(None, 4, 128, FAKE, None) == EINVAL
    q = L.nvfp4_quantize_sr
    assert q(FAKE, 1, 64, 48, 1, 7, FAKE, FAKE, FAKE, None) == EUNSUP              # cols % 32
    assert q(FAKE, 3, 64, 256, 1, 7, FAKE, FAKE, FAKE, None) == EINVAL             # dtype
    assert q(None, 1, 64, 256, 1, 7, FAKE, FAKE, FAKE, None) == EINVAL
    r = L.nvfp4_requant_sr
    args = lambda mode, rpg, cols, P, layout: (FAKE, FAKE, FAKE, mode, rpg, 64, cols, FAKE, FAKE, 2,
                                               P, layout, 1, 5, FAKE, FAKE, FAKE, None)
    assert r(*args(2, 0, 256, 256, 0)) == EINVAL                                   # outer mode
    assert r(*args(1, 0, 256, 256, 0)) == EINVAL                                   # rows_per_group
    assert r(*args(0, 0, 256, 256, 5)) == EINVAL                                   # layout
    assert r(*args(0, 0, 192, 256, 0)) == EUNSUP                                   # cols % 128
    assert r(*args(0, 0, 256, 96, 0)) == EUNSUP                                    # P % 128
    c = L.nvfp4_quantize_sr_colwise
    assert c(FAKE, 1, 64, 256, None, FAKE, 2, 256, 1, 8, FAKE, FAKE, FAKE, None) == EINVAL
    assert c(FAKE, 1, 64, 200, FAKE, FAKE, 2, 256, 1, 8, FAKE, FAKE, FAKE, None) == EUNSUP
    w = L.moe_bwd_wgrad_nvfp4
    wa = lambda P, N, K: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, P, N, K, FAKE, None)
    assert w(*wa(256, 384, 256)) == EUNSUP                                         # N % 256
    assert w(*wa(256, 256, 128)) == EUNSUP                                         # K % 256
    assert w(*wa(200, 256, 256)) == EUNSUP                                         # P % 128
    assert w(*wa(1 << 26, 256, 256)) == EUNSUP                                     # 32-bit range
    assert w(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, 256, FAKE, None) == EINVAL


def test_binding_rejects_host_tensors():
    import torch
    from precision_moe_numerics_nvfp4_amd import binding
    ensure_built()
    with pytest.raises(ValueError):
        binding.nvfp4_quantize(torch.zeros(4, 64))
    with pytest.raises(TypeError):
        binding.nvfp4_quantize([[0.0] * 64])
