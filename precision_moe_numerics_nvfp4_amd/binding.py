"""ctypes binding of libnvfp4moe.so (see include/nvfp4moe.h for the contract).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch (device memory), the current stream, and status-code -> exception.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4moe.so")

NVFP4MOE_F32 = 0
NVFP4MOE_BF16 = 1
_OUTER_PER_ROW, _OUTER_PER_GROUP = 0, 1
_LAYOUT_TRANSPOSED, _LAYOUT_PER_GROUP = 0, 1
_ROWWISE, _COLWISE_GROUPED = 0, 1

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_u32 = ctypes.c_uint32
_c_u64 = ctypes.c_uint64
_c_size = ctypes.c_size_t
_p = ctypes.c_void_p

# name -> argument types (all return int status, except where noted)
SIGNATURES = {
    "nvfp4moe_abi_version": ([], _c_int),
    "nvfp4moe_status_string": ([_c_int], ctypes.c_char_p),
    "nvfp4_quantize": ([_p, _c_int, _c_i64, _c_i64, _c_int, _c_i64, _p, _p, _p, _p], _c_int),
    "nvfp4moe_permute_workspace_size": ([_c_i64, _c_int, _c_int], _c_size),
    "moe_permute": ([_p, _c_i64, _c_int, _c_int, _c_int, _p, _p, _p, _c_i64, _p, _p, _p, _p,
                     _p, _p, _p, _p, _p, _c_size, _p], _c_int),
    "moe_permute_noalloc": ([_p, _c_i64, _c_int, _c_int, _c_int, _p, _p, _p, _c_i64, _p, _p, _p,
                             _p, _p, _p, _p, _p, _p], _c_int),
    "moe_fwd_grouped_gemm": ([_p, _p, _p, _p, _p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p,
                              _c_int, _p], _c_int),
    "mxfp8_requant_sr": ([_p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p, _p, _c_int, _c_i64,
                          _c_u64, _c_u32, _p, _p, _p], _c_int),
    "mxfp8_quantize": ([_p, _c_int, _c_i64, _c_i64, _c_int, _p, _p, _c_int, _c_i64, _p, _p, _p],
                       _c_int),
    "moe_bwd_dgrad": ([_p, _p, _p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p, _c_int, _p],
                      _c_int),
    "moe_bwd_wgrad": ([_p, _p, _p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p, _p], _c_int),
    "moe_fwd_grouped_gemm_mxfp8": ([_p, _p, _p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p,
                                    _c_int, _p], _c_int),
    "mxfp8_gather_rows": ([_p, _p, _c_int, _c_i64, _p, _p, _c_i64, _c_i64, _p, _p, _p], _c_int),
    "nvfp4_quantize_tile16": ([_p, _c_int, _c_i64, _c_i64, _c_i64, _p, _p, _p, _p], _c_int),
    "mxfp8_quantize_dual": ([_p, _c_int, _c_i64, _c_i64, _p, _p, _c_int, _c_i64, _p, _p, _p, _p,
                             _p], _c_int),
    "nvfp4_quantize_live": ([_p, _c_int, _c_i64, _c_i64, _p, _p, _p, _p, _p], _c_int),
    "moe_combine": ([_p, _c_int, _c_i64, _c_i64, _c_int, _c_i64, _p, _p, _p, _c_int, _p], _c_int),
    "moe_combine_bwd": ([_p, _c_int, _c_i64, _c_int, _c_i64, _p, _p, _p, _c_int, _c_i64, _p, _p,
                         _c_int, _p, _c_int, _p, _p], _c_int),
    "moe_padded_offsets": ([_p, _c_int, _c_int, _p, _p], _c_int),
    "nvfp4_quantize_sr": ([_p, _c_int, _c_i64, _c_i64, _c_u64, _c_u32, _p, _p, _p, _p], _c_int),
    "nvfp4_requant_sr": ([_p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p, _p, _c_int, _c_i64,
                          _c_int, _c_u64, _c_u32, _p, _p, _p, _p], _c_int),
    "nvfp4_quantize_sr_colwise": ([_p, _c_int, _c_i64, _c_i64, _p, _p, _c_int, _c_i64, _c_u64,
                                   _c_u32, _p, _p, _p, _p], _c_int),
    "moe_bwd_wgrad_nvfp4": ([_p, _p, _p, _p, _p, _p, _p, _c_int, _c_i64, _c_i64, _c_i64, _p, _p],
                            _c_int),
}

_LIB = None


class Nvfp4moeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def lib():
    """Load libnvfp4moe.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m precision_moe_numerics_nvfp4_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def abi_version():
    return lib().nvfp4moe_abi_version()


def status_string(status):
    return lib().nvfp4moe_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise Nvfp4moeError(fn, status)


def _torch():
    import torch
    return torch


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _in_dtype(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return NVFP4MOE_F32
    if x.dtype == torch.bfloat16:
        return NVFP4MOE_BF16
    raise ValueError(f"input must be float32 or bfloat16 (got {x.dtype})")


def _out_dtype(dtype):
    torch = _torch()
    if dtype == torch.float32:
        return NVFP4MOE_F32
    if dtype == torch.bfloat16:
        return NVFP4MOE_BF16
    raise ValueError(f"output dtype must be float32 or bfloat16 (got {dtype})")


def nvfp4_quantize(x, rows_per_group=None, codes=None, scales=None, outer=None):
    """x [rows, cols] float32|bfloat16 -> (codes [rows, cols/2] u8, scales
    [rows, cols/16] u8, outer f32 [rows] or [rows/rows_per_group])."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    n_outer = rows if rows_per_group is None else rows // max(int(rows_per_group), 1)
    if outer is None:
        outer = torch.empty((n_outer,), dtype=torch.float32, device=dev)
    mode = _OUTER_PER_ROW if rows_per_group is None else _OUTER_PER_GROUP
    st = lib().nvfp4_quantize(_ptr(x), _in_dtype(x), rows, cols, mode,
                              0 if rows_per_group is None else int(rows_per_group),
                              _ptr(codes), _ptr(scales), _ptr(outer), _stream(x))
    _check("nvfp4_quantize", st)
    return codes, scales, outer


def permute_workspace_size(T, k, n_local):
    return int(lib().nvfp4moe_permute_workspace_size(int(T), int(k), int(n_local)))


def moe_permute(topk_ids, e0, n_local, xq_codes, xq_scales, xq_outer, workspace=None, out=None):
    """Group routed (token, slot) pairs by local expert and gather NVFP4 rows.

    Returns a dict with offsets, padded_offsets (int64 [n_local+1]), row_token,
    row_slot (int32 [T*k]), pair_row (int32 [T, k], the row of each pair or
    -1) and codes/scales/outer of the permuted rows (capacity T*k rows; rows
    >= offsets[-1] are not written). An ``out`` dict without "pair_row" asks
    for no inverse map."""
    torch = _torch()
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    _dev(xq_codes, "xq_codes", torch.uint8, 2)
    _dev(xq_scales, "xq_scales", torch.uint8, 2)
    _dev(xq_outer, "xq_outer", torch.float32, 1)
    K = xq_codes.shape[1] * 2
    dev = topk_ids.device
    cap = T * k
    o = dict(out or {})
    if out is None:
        o["pair_row"] = torch.empty((T, k), dtype=torch.int32, device=dev)
    o.setdefault("offsets", torch.empty((n_local + 1,), dtype=torch.int64, device=dev))
    o.setdefault("padded_offsets", torch.empty((n_local + 1,), dtype=torch.int64, device=dev))
    o.setdefault("row_token", torch.empty((cap,), dtype=torch.int32, device=dev))
    o.setdefault("row_slot", torch.empty((cap,), dtype=torch.int32, device=dev))
    o.setdefault("codes", torch.empty((cap, K // 2), dtype=torch.uint8, device=dev))
    o.setdefault("scales", torch.empty((cap, K // 16), dtype=torch.uint8, device=dev))
    o.setdefault("outer", torch.empty((cap,), dtype=torch.float32, device=dev))
    ws_bytes = permute_workspace_size(T, k, n_local)
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    st = lib().moe_permute(_ptr(topk_ids), T, k, int(e0), int(n_local), _ptr(xq_codes),
                           _ptr(xq_scales), _ptr(xq_outer), K, _ptr(o["offsets"]),
                           _ptr(o["padded_offsets"]), _ptr(o["row_token"]), _ptr(o["row_slot"]),
                           _ptr(o.get("pair_row")), _ptr(o["codes"]), _ptr(o["scales"]), _ptr(o["outer"]),
                           _ptr(workspace), workspace.numel(), _stream(topk_ids))
    _check("moe_permute", st)
    return o


def moe_permute_noalloc(topk_ids, e0, n_local, xq_codes, xq_scales, xq_outer, out):
    """moe_permute through the entry point that allocates nothing: the
    library keeps the count table in its own per-GPU array (at most 4 MiB,
    see the header), and every output buffer comes from the caller in `out`
    (the dict moe_permute returns or takes; "pair_row" optional)."""
    torch = _torch()
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    _dev(xq_codes, "xq_codes", torch.uint8, 2)
    _dev(xq_scales, "xq_scales", torch.uint8, 2)
    _dev(xq_outer, "xq_outer", torch.float32, 1)
    K = xq_codes.shape[1] * 2
    for name in ("offsets", "padded_offsets", "row_token", "row_slot", "codes", "scales", "outer"):
        if name not in out:
            raise ValueError(f"moe_permute_noalloc: out lacks {name}")
    st = lib().moe_permute_noalloc(_ptr(topk_ids), T, k, int(e0), int(n_local), _ptr(xq_codes),
                                   _ptr(xq_scales), _ptr(xq_outer), K, _ptr(out["offsets"]),
                                   _ptr(out["padded_offsets"]), _ptr(out["row_token"]),
                                   _ptr(out["row_slot"]), _ptr(out.get("pair_row")),
                                   _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["outer"]),
                                   _stream(topk_ids))
    _check("moe_permute_noalloc", st)
    return out


def moe_fwd_grouped_gemm(a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, offsets,
                         out_dtype=None, y=None):
    """y [m_cap, N] = grouped NVFP4 GEMM (see the header). b_* are [G*N, ...]
    or [G, N, ...]; offsets int64 [G+1] on the device."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    _dev(a_codes, "a_codes", torch.uint8, 2)
    _dev(a_scales, "a_scales", torch.uint8, 2)
    _dev(a_outer, "a_outer", torch.float32, 1)
    _dev(b_codes, "b_codes", torch.uint8)
    _dev(b_scales, "b_scales", torch.uint8)
    _dev(b_outer, "b_outer", torch.float32, 1)
    _dev(offsets, "offsets", torch.int64, 1)
    m_cap, K = a_codes.shape[0], a_codes.shape[1] * 2
    G = b_outer.shape[0]
    N = b_codes.numel() // (G * (K // 2)) if G else 0
    if y is None:
        y = torch.empty((m_cap, N), dtype=out_dtype, device=a_codes.device)
    st = lib().moe_fwd_grouped_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_outer), _ptr(b_codes),
                                    _ptr(b_scales), _ptr(b_outer), _ptr(offsets), G, m_cap, N, K,
                                    _ptr(y), _out_dtype(y.dtype), _stream(a_codes))
    _check("moe_fwd_grouped_gemm", st)
    return y


def mxfp8_requant_sr(codes, scales, outer, offsets, padded_offsets, P, seed, tag,
                     rows_per_group=None, out=None, out_e8=None):
    """Saved NVFP4 [rows, cols] -> MXFP8 with stochastic rounding, grouped
    transpose per offsets/padded_offsets: activations (per-row outer scales)
    [cols, P] (+ E8M0 [cols, P/32]); weights (rows_per_group) per-expert blocks
    [G * cols, rows_per_group] (+ [G * cols, rows_per_group/32]), P = G *
    rows_per_group."""
    torch = _torch()
    _dev(codes, "codes", torch.uint8, 2)
    _dev(scales, "scales", torch.uint8, 2)
    _dev(outer, "outer", torch.float32, 1)
    _dev(offsets, "offsets", torch.int64, 1)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    G = offsets.shape[0] - 1
    dev = codes.device
    if rows_per_group is None:
        shape = (cols, P)
    else:
        if P != G * rows_per_group:
            raise ValueError("mxfp8_requant_sr: weights need P == G * rows_per_group")
        shape = (G * cols, rows_per_group)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=dev)
    if out_e8 is None:
        out_e8 = torch.empty((shape[0], shape[1] // 32), dtype=torch.uint8, device=dev)
    if out.numel() < shape[0] * shape[1] or out_e8.numel() < shape[0] * (shape[1] // 32):
        raise ValueError("mxfp8_requant_sr: output buffers too small")
    mode = _OUTER_PER_ROW if rows_per_group is None else _OUTER_PER_GROUP
    st = lib().mxfp8_requant_sr(_ptr(codes), _ptr(scales), _ptr(outer), mode,
                                0 if rows_per_group is None else int(rows_per_group), rows, cols,
                                _ptr(offsets), _ptr(padded_offsets), G, int(P),
                                int(seed) & 0xFFFFFFFFFFFFFFFF, int(tag) & 0xFFFFFFFF,
                                _ptr(out), _ptr(out_e8), _stream(codes))
    _check("mxfp8_requant_sr", st)
    return out, out_e8


def mxfp8_quantize(x, orientation="rowwise", offsets=None, padded_offsets=None, P=0,
                   out=None, out_e8=None):
    """dY [rows, cols] float32|bfloat16 -> MXFP8 with round-to-nearest-even.
    'rowwise': [rows, cols] + [rows, cols/32]; 'colwise': grouped transpose
    [cols, P] + [cols, P/32]."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    rows, cols = x.shape
    dev = x.device
    if orientation == "rowwise":
        if out is None:
            out = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        if out_e8 is None:
            out_e8 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        st = lib().mxfp8_quantize(_ptr(x), _in_dtype(x), rows, cols, _ROWWISE, None, None, 0, 0,
                                  _ptr(out), _ptr(out_e8), _stream(x))
    elif orientation == "colwise":
        _dev(offsets, "offsets", torch.int64, 1)
        _dev(padded_offsets, "padded_offsets", torch.int64, 1)
        G = offsets.shape[0] - 1
        if out is None:
            out = torch.empty((cols, P), dtype=torch.uint8, device=dev)
        if out_e8 is None:
            out_e8 = torch.empty((cols, P // 32), dtype=torch.uint8, device=dev)
        st = lib().mxfp8_quantize(_ptr(x), _in_dtype(x), rows, cols, _COLWISE_GROUPED,
                                  _ptr(offsets), _ptr(padded_offsets), G, int(P), _ptr(out),
                                  _ptr(out_e8), _stream(x))
    else:
        raise ValueError("orientation must be 'rowwise' or 'colwise'")
    _check("mxfp8_quantize", st)
    return out, out_e8


def moe_bwd_dgrad(dy_e4m3, dy_e8m0, w_e4m3, w_e8m0, offsets, N, K, out_dtype=None, dx=None):
    """dX [m_cap, K] from dY8 [m_cap, N] and W8 [G*K, N] (MXFP8, each expert's
    transposed weight [K, N] contiguous, as mxfp8_requant_sr writes it)."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    for t, n in ((dy_e4m3, "dy_e4m3"), (dy_e8m0, "dy_e8m0"), (w_e4m3, "w_e4m3"),
                 (w_e8m0, "w_e8m0")):
        _dev(t, n, torch.uint8, 2)
    _dev(offsets, "offsets", torch.int64, 1)
    m_cap = dy_e4m3.shape[0]
    G = offsets.shape[0] - 1
    if dx is None:
        dx = torch.empty((m_cap, K), dtype=out_dtype, device=dy_e4m3.device)
    st = lib().moe_bwd_dgrad(_ptr(dy_e4m3), _ptr(dy_e8m0), _ptr(w_e4m3), _ptr(w_e8m0),
                             _ptr(offsets), G, m_cap, int(N), int(K), _ptr(dx),
                             _out_dtype(dx.dtype), _stream(dy_e4m3))
    _check("moe_bwd_dgrad", st)
    return dx


def moe_bwd_wgrad(dyT_e4m3, dyT_e8m0, xT_e4m3, xT_e8m0, padded_offsets, N, K, dw=None):
    """dW [G, N, K] float32 from dYT8 [N, P] and XT8 [K, P] (MXFP8)."""
    torch = _torch()
    for t, n in ((dyT_e4m3, "dyT_e4m3"), (dyT_e8m0, "dyT_e8m0"), (xT_e4m3, "xT_e4m3"),
                 (xT_e8m0, "xT_e8m0")):
        _dev(t, n, torch.uint8, 2)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    G = padded_offsets.shape[0] - 1
    P = dyT_e4m3.shape[1]
    if dw is None:
        dw = torch.empty((G, N, K), dtype=torch.float32, device=dyT_e4m3.device)
    st = lib().moe_bwd_wgrad(_ptr(dyT_e4m3), _ptr(dyT_e8m0), _ptr(xT_e4m3), _ptr(xT_e8m0),
                             _ptr(padded_offsets), G, P, int(N), int(K), _ptr(dw),
                             _stream(dyT_e4m3))
    _check("moe_bwd_wgrad", st)
    return dw


def moe_fwd_grouped_gemm_mxfp8(x_e4m3, x_e8m0, w_e4m3, w_e8m0, offsets, out_dtype=None, y=None):
    """y [m_cap, N] from X8 [m_cap, K] and weights W8 [G*N, K] or [G, N, K] (MXFP8)."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    _dev(x_e4m3, "x_e4m3", torch.uint8, 2)
    _dev(x_e8m0, "x_e8m0", torch.uint8, 2)
    _dev(w_e4m3, "w_e4m3", torch.uint8)
    _dev(w_e8m0, "w_e8m0", torch.uint8)
    _dev(offsets, "offsets", torch.int64, 1)
    m_cap, K = x_e4m3.shape
    G = offsets.shape[0] - 1
    N = (w_e4m3.numel() // K) // G if G else 0
    if w_e4m3.numel() != G * N * K or w_e8m0.numel() != G * N * (K // 32):
        raise ValueError("weights must hold G*N rows of K elements (and K/32 scales)")
    if y is None:
        y = torch.empty((m_cap, N), dtype=out_dtype, device=x_e4m3.device)
    st = lib().moe_fwd_grouped_gemm_mxfp8(_ptr(x_e4m3), _ptr(x_e8m0), _ptr(w_e4m3), _ptr(w_e8m0),
                                          _ptr(offsets), G, m_cap, N, K, _ptr(y),
                                          _out_dtype(y.dtype), _stream(x_e4m3))
    _check("moe_fwd_grouped_gemm_mxfp8", st)
    return y


def mxfp8_gather_rows(row_token, offsets, src_e4m3, src_e8m0, m_cap=None, out=None):
    """Rows of MXFP8 src [T, K] (+ [T, K/32]) in expert order: row r < offsets[-1]
    is src row row_token[r]. Returns (dst_e4m3 [m_cap, K], dst_e8m0 [m_cap, K/32])."""
    torch = _torch()
    _dev(row_token, "row_token", torch.int32, 1)
    _dev(offsets, "offsets", torch.int64, 1)
    _dev(src_e4m3, "src_e4m3", torch.uint8, 2)
    _dev(src_e8m0, "src_e8m0", torch.uint8, 2)
    T, K = src_e4m3.shape
    m_cap = row_token.shape[0] if m_cap is None else int(m_cap)
    if out is None:
        out = (torch.empty((m_cap, K), dtype=torch.uint8, device=src_e4m3.device),
               torch.empty((m_cap, K // 32), dtype=torch.uint8, device=src_e4m3.device))
    G = offsets.shape[0] - 1
    st = lib().mxfp8_gather_rows(_ptr(row_token), _ptr(offsets), G, m_cap, _ptr(src_e4m3),
                                 _ptr(src_e8m0), T, K, _ptr(out[0]), _ptr(out[1]),
                                 _stream(src_e4m3))
    _check("mxfp8_gather_rows", st)
    return out


def mxfp8_quantize_dual(x, offsets, padded_offsets, P, row_out=None, col_out=None):
    """dY [rows, cols] -> (row-wise MXFP8 [rows, cols] + [rows, cols/32] for the
    grouped rows, grouped column-wise [cols, P] + [cols, P/32]) in one pass."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    _dev(offsets, "offsets", torch.int64, 1)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    rows, cols = x.shape
    dev = x.device
    if row_out is None:
        row_out = (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                   torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev))
    if col_out is None:
        col_out = (torch.empty((cols, P), dtype=torch.uint8, device=dev),
                   torch.empty((cols, P // 32), dtype=torch.uint8, device=dev))
    G = offsets.shape[0] - 1
    st = lib().mxfp8_quantize_dual(_ptr(x), _in_dtype(x), rows, cols, _ptr(offsets),
                                   _ptr(padded_offsets), G, int(P), _ptr(row_out[0]),
                                   _ptr(row_out[1]), _ptr(col_out[0]), _ptr(col_out[1]), _stream(x))
    _check("mxfp8_quantize_dual", st)
    return row_out[0], row_out[1], col_out[0], col_out[1]


def nvfp4_quantize_tile16(x, rows_per_group=None, codes=None, scales=None, outer=None):
    """16x16-tile NVFP4 of x [rows, cols] (bf16|f32): (codes [rows, cols/2],
    scales [rows/16, cols/16], outer [rows/rows_per_group])."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    rows, cols = x.shape
    rpg = rows if rows_per_group is None else int(rows_per_group)
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows // 16, cols // 16), dtype=torch.uint8, device=dev)
    if outer is None:
        outer = torch.empty((max(rows // max(rpg, 1), 1),), dtype=torch.float32, device=dev)
    st = lib().nvfp4_quantize_tile16(_ptr(x), _in_dtype(x), rows, cols, rpg, _ptr(codes),
                                     _ptr(scales), _ptr(outer), _stream(x))
    _check("nvfp4_quantize_tile16", st)
    return codes, scales, outer


def nvfp4_quantize_live(x, offsets, codes=None, scales=None, outer=None):
    """Per-row NVFP4 of the routed rows r < offsets[-1] of x [m_cap, cols]
    (bf16|f32): (codes [m_cap, cols/2], scales [m_cap, cols/16], outer
    [m_cap]); later rows untouched."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    _dev(offsets, "offsets", torch.int64, 1)
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if outer is None:
        outer = torch.empty((rows,), dtype=torch.float32, device=dev)
    st = lib().nvfp4_quantize_live(_ptr(x), _in_dtype(x), rows, cols, _ptr(offsets[-1:]),
                                   _ptr(codes), _ptr(scales), _ptr(outer), _stream(x))
    _check("nvfp4_quantize_live", st)
    return codes, scales, outer


def moe_combine(y, pair_row, gate=None, out_dtype=None, out=None):
    """out [T, N] = sum_j gate[t, j] * y[pair_row[t, j]] (gate None: ones).
    y [m_cap, N] bf16|f32; pair_row int32 [T, k]; gate f32 [T, k]."""
    torch = _torch()
    _dev(y, "y", ndim=2)
    _dev(pair_row, "pair_row", torch.int32, 2)
    if gate is not None:
        _dev(gate, "gate", torch.float32, 2)
        if tuple(gate.shape) != tuple(pair_row.shape):
            raise ValueError("gate and pair_row must have the same shape")
    T, k = pair_row.shape
    N = y.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype or y.dtype, device=y.device)
    _dev(out, "out", ndim=2)
    st = lib().moe_combine(_ptr(y), _in_dtype(y), y.shape[0], T, k, N, _ptr(pair_row),
                           _ptr(gate), _ptr(out), _out_dtype(out.dtype), _stream(y))
    _check("moe_combine", st)
    return out


def moe_combine_bwd(dout, row_token, row_slot, offsets, k, gate=None, y=None, dy=None,
                    dgate=None, dy_dtype=None, m_cap=None):
    """Backward of moe_combine for the routed rows: (dy [m_cap, N], dgate
    [T, k] or None). dout [T, N]; y [m_cap, N] (the forward's expert outputs)
    or None; rows >= offsets[-1] of dy and non-local dgate entries untouched."""
    torch = _torch()
    _dev(dout, "dout", ndim=2)
    _dev(row_token, "row_token", torch.int32, 1)
    _dev(row_slot, "row_slot", torch.int32, 1)
    _dev(offsets, "offsets", torch.int64, 1)
    T, N = dout.shape
    if m_cap is None:
        m_cap = row_token.shape[0] if dy is None else dy.shape[0]
    if dy is None:
        dy = torch.empty((m_cap, N), dtype=dy_dtype or dout.dtype, device=dout.device)
    _dev(dy, "dy", ndim=2)
    if gate is not None:
        _dev(gate, "gate", torch.float32, 2)
    if y is not None:
        _dev(y, "y", ndim=2)
        if dgate is None:
            dgate = torch.zeros((T, k), dtype=torch.float32, device=dout.device)
    G = offsets.shape[0] - 1
    st = lib().moe_combine_bwd(_ptr(dout), _in_dtype(dout), T, int(k), N, _ptr(row_token),
                               _ptr(row_slot), _ptr(offsets), G, int(m_cap), _ptr(gate), _ptr(y),
                               _in_dtype(y) if y is not None else NVFP4MOE_F32, _ptr(dy),
                               _out_dtype(dy.dtype), _ptr(dgate), _stream(dout))
    _check("moe_combine_bwd", st)
    return dy, dgate


# ------------------------------------------------------------ NVFP4 backward

def moe_padded_offsets(offsets, align=128, out=None):
    """Exclusive scan of the group lengths rounded up to ``align`` (int64 [G+1])."""
    torch = _torch()
    _dev(offsets, "offsets", torch.int64, 1)
    G = offsets.shape[0] - 1
    if out is None:
        out = torch.empty_like(offsets)
    st = lib().moe_padded_offsets(_ptr(offsets), G, int(align), _ptr(out), _stream(offsets))
    _check("moe_padded_offsets", st)
    return out


def nvfp4_quantize_sr(x, seed, tag, codes=None, scales=None, outer=None):
    """Row-wise NVFP4 of x [rows, cols] with stochastic rounding and rounded-up
    block scales: (codes [rows, cols/2], scales [rows, cols/16], outer [rows])."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if outer is None:
        outer = torch.empty((rows,), dtype=torch.float32, device=dev)
    st = lib().nvfp4_quantize_sr(_ptr(x), _in_dtype(x), rows, cols, int(seed), int(tag),
                                 _ptr(codes), _ptr(scales), _ptr(outer), _stream(x))
    _check("nvfp4_quantize_sr", st)
    return codes, scales, outer


def nvfp4_requant_sr(codes, scales, outer, offsets, padded_offsets, P, seed, tag,
                     rows_per_group=None, per_group_layout=False, out=None):
    """Saved NVFP4 [rows, cols] -> grouped transpose -> NVFP4 with stochastic
    rounding, one outer scale per group. Transposed layout: (codes [cols, P/2],
    scales [cols, P/16], outer [G]); per-group layout (groups of one length L,
    P = G * L): (codes [G * cols, L/2], scales [G * cols, L/16], outer [G])."""
    torch = _torch()
    _dev(codes, "codes", torch.uint8, 2)
    _dev(scales, "scales", torch.uint8, 2)
    _dev(outer, "outer", torch.float32, 1)
    _dev(offsets, "offsets", torch.int64, 1)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    G = offsets.shape[0] - 1
    dev = codes.device
    if out is None:
        if per_group_layout:
            L = P // max(G, 1)
            out = (torch.empty((G * cols, L // 2), dtype=torch.uint8, device=dev),
                   torch.empty((G * cols, L // 16), dtype=torch.uint8, device=dev),
                   torch.empty((G,), dtype=torch.float32, device=dev))
        else:
            out = (torch.empty((cols, P // 2), dtype=torch.uint8, device=dev),
                   torch.empty((cols, P // 16), dtype=torch.uint8, device=dev),
                   torch.empty((G,), dtype=torch.float32, device=dev))
    mode = _OUTER_PER_ROW if rows_per_group is None else _OUTER_PER_GROUP
    st = lib().nvfp4_requant_sr(_ptr(codes), _ptr(scales), _ptr(outer), mode,
                                0 if rows_per_group is None else int(rows_per_group), rows, cols,
                                _ptr(offsets), _ptr(padded_offsets), G, int(P),
                                _LAYOUT_PER_GROUP if per_group_layout else _LAYOUT_TRANSPOSED,
                                int(seed), int(tag), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                _stream(codes))
    _check("nvfp4_requant_sr", st)
    return out


def nvfp4_quantize_sr_colwise(x, offsets, padded_offsets, P, seed, tag, out=None):
    """dY [rows, cols] -> grouped transpose [cols, P] -> NVFP4 with stochastic
    rounding, one outer scale per group: (codes [cols, P/2], scales
    [cols, P/16], outer [G])."""
    torch = _torch()
    _dev(x, "x", ndim=2)
    _dev(offsets, "offsets", torch.int64, 1)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    rows, cols = x.shape
    G = offsets.shape[0] - 1
    dev = x.device
    if out is None:
        out = (torch.empty((cols, P // 2), dtype=torch.uint8, device=dev),
               torch.empty((cols, P // 16), dtype=torch.uint8, device=dev),
               torch.empty((G,), dtype=torch.float32, device=dev))
    st = lib().nvfp4_quantize_sr_colwise(_ptr(x), _in_dtype(x), rows, cols, _ptr(offsets),
                                         _ptr(padded_offsets), G, int(P), int(seed), int(tag),
                                         _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(x))
    _check("nvfp4_quantize_sr_colwise", st)
    return out


def moe_bwd_wgrad_nvfp4(dyT, xT, padded_offsets, N, K, dw=None):
    """dW [G, N, K] float32 from NVFP4 dYT [N, P] and XT [K, P], each given as
    (codes, scales, outer [G])."""
    torch = _torch()
    for t, n in ((dyT[0], "dyT codes"), (dyT[1], "dyT scales"), (xT[0], "xT codes"),
                 (xT[1], "xT scales")):
        _dev(t, n, torch.uint8, 2)
    _dev(dyT[2], "dyT outer", torch.float32, 1)
    _dev(xT[2], "xT outer", torch.float32, 1)
    _dev(padded_offsets, "padded_offsets", torch.int64, 1)
    G = padded_offsets.shape[0] - 1
    P = dyT[0].shape[1] * 2
    if dw is None:
        dw = torch.empty((G, N, K), dtype=torch.float32, device=dyT[0].device)
    st = lib().moe_bwd_wgrad_nvfp4(_ptr(dyT[0]), _ptr(dyT[1]), _ptr(dyT[2]), _ptr(xT[0]),
                                   _ptr(xT[1]), _ptr(xT[2]), _ptr(padded_offsets), G, P, int(N),
                                   int(K), _ptr(dw), _stream(dyT[0]))
    _check("moe_bwd_wgrad_nvfp4", st)
    return dw
