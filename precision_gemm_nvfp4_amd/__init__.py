"""Python binding of libnvfp4_resq.so: the MI355X NVFP4 W4A4 MoE expert GEMM
with residual activation compensation, weight QDQ and rollout-guided
rounding.

Argument marshalling only: every step runs in the HIP library.  torch
provides device memory (outputs and workspaces are torch tensors) and the
stream (torch.cuda.current_stream()).  The functions carry the C ABI's names;
see include/nvfp4_resq.h for the contract of each.  There is no CPU fallback:
without the built library every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_resq.so")

NVFP4_DTYPE_BF16 = 0
NVFP4_DTYPE_F32 = 1
EPI_F32 = 0
EPI_SWIGLU_BF16 = 1
EPI_SCATTER_ADD_F32 = 2
EPI_SCATTER_F32 = 3

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "nvfp4_version": (_INT, []),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_quantize_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_quantize_noalloc": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "resq_select_and_requant_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "resq_select_and_requant": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64,
                                       _I64, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "resq_mask_select_and_requant": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                                            _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_w4a4_masked_comp_gemm": (_INT, [_P, _P, _P, _P, _I32, _I64, _I64, _P, _P, _P, _I64, _P,
                                         _I64, _P]),
    "moe_w4a4_grouped_gemm_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _INT, _I64]),
    "moe_w4a4_grouped_gemm": (_INT, [_P, _P, _P, _P, _I64, _P, _I32, _I64, _I64, _P, _P, _P,
                                     _I64, _P, _P, _P, _P, _I32, _INT, _P, _P, _I64, _P, _I64,
                                     _P, _P, _SZ, _P]),
    "qdq_weights_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "qdq_weights": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "guided_round": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "guidance_record_pack": (_INT, [_P, _I64, _I64, _P, _P]),
    "guided_round_record": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "mxfp4_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P]),
    "mxfp4_resq_select_and_requant_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "mxfp4_resq_select_and_requant": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _I64,
                                             _I64, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_grouped_gemm_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _INT, _I64]),
    "moe_mxfp4_grouped_gemm": (_INT, [_P, _P, _P, _I64, _P, _I32, _I64, _I64, _P, _P, _I64,
                                      _P, _P, _P, _I32, _INT, _P, _P, _I64, _P, _I64, _P, _P,
                                      _SZ, _P]),
    "mxfp4_qdq_weights": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "mxfp4_guided_round": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "mxfp4_guided_round_record": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "mxfp8_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P]),
    "moe_mxfp4_w4a8_grouped_gemm_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _INT, _I64]),
    "moe_mxfp4_w4a8_grouped_gemm": (_INT, [_P, _P, _P, _I64, _P, _I32, _I64, _I64, _P, _P, _I64,
                                           _INT, _P, _P, _I64, _P, _I64, _P, _P, _SZ, _P]),
}


def load():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m precision_gemm_nvfp4_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def _check(status, name):
    if status != 0:
        msg = load().nvfp4_last_error().decode()
        raise RuntimeError(f"{name} failed with status {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return NVFP4_DTYPE_BF16
    if t.dtype == torch.float32:
        return NVFP4_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


# ---------------------------------------------------------------------------
def nvfp4_quantize(x, amax_in=None, tile_partials=False):
    """NVFP4 quantization of x [M, K] (bf16/fp32, GPU).

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/16], g fp32 [1],
    tile_partials fp32 [ceil(M/128), K] or None)."""
    lib = load()
    _require_cuda(x, amax_in)
    m, k = x.shape
    dev = x.device
    codes = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(m, k // 16, dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    tp = torch.empty((m + 127) // 128, k, dtype=torch.float32, device=dev) if tile_partials else None
    ws_n = lib.nvfp4_quantize_workspace_size(m, k)
    ws = _workspace(ws_n, dev)
    _check(lib.nvfp4_quantize(_ptr(x), _dtype_code(x), m, k, x.stride(0), _ptr(amax_in),
                              _ptr(codes), _ptr(scales), _ptr(g), _ptr(tp), _ptr(ws), ws.numel(),
                              _stream()), "nvfp4_quantize")
    return codes, scales, g, tp


def nvfp4_quantize_noalloc(x, codes, scales, g, amax_in=None, tile_partials=None):
    """nvfp4_quantize into caller-given outputs, with the library's own
    per-device scratch instead of a workspace: this call allocates nothing.

    codes uint8 [M, K/2], scales uint8 [M, K/16], g fp32 [1] (or None),
    tile_partials fp32 [ceil(M/128), K] or None; all on the GPU."""
    lib = load()
    _require_cuda(x, codes, scales, g, amax_in, tile_partials)
    m, k = x.shape
    _check(lib.nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x), m, k, x.stride(0), _ptr(amax_in),
                                      _ptr(codes), _ptr(scales), _ptr(g), _ptr(tile_partials),
                                      _stream()), "nvfp4_quantize_noalloc")
    return codes, scales, g, tile_partials


def resq_select_and_requant(x, codes, scales, g, k, unit_offsets=None, rows_total=None,
                            row_index=None, tile_partials=None):
    """Select the top-k residual channels of each unit and requantize R_S.

    unit_offsets: int64 GPU tensor [U+1] (with rows_total = its last value as
    a host int), or None with tile_partials from nvfp4_quantize (units = the
    128-row tiles of x).  Returns (sel_idx int32 [U, k], r_codes [rows, k/2],
    r_scales [rows, k/16], r_global fp32 [U])."""
    lib = load()
    _require_cuda(x, codes, scales, g, unit_offsets, row_index, tile_partials)
    x_rows, kk = x.shape
    dev = x.device
    if tile_partials is not None:
        n_units = (x_rows + 127) // 128
        rows_total = x_rows
    else:
        n_units = unit_offsets.numel() - 1
        if rows_total is None:
            raise ValueError("rows_total (host int) is required with unit_offsets")
    sel = torch.empty(n_units, k, dtype=torch.int32, device=dev)
    rc = torch.empty(rows_total, k // 2, dtype=torch.uint8, device=dev)
    rs = torch.empty(rows_total, k // 16, dtype=torch.uint8, device=dev)
    rg = torch.empty(n_units, dtype=torch.float32, device=dev)
    ws = _workspace(lib.resq_select_and_requant_workspace_size(kk, rows_total, n_units, k), dev)
    _check(lib.resq_select_and_requant(
        _ptr(x), _dtype_code(x), x_rows, kk, x.stride(0), _ptr(row_index), _ptr(codes),
        _ptr(scales), _ptr(g), _ptr(unit_offsets), n_units, rows_total, k, _ptr(tile_partials),
        _ptr(sel), _ptr(rc), _ptr(rs), _ptr(rg), _ptr(ws), ws.numel(), _stream()),
        "resq_select_and_requant")
    return sel, rc, rs, rg


def resq_mask_select_and_requant(x, codes, scales, g, k, unit_offsets=None, rows_total=None,
                                 row_index=None, tile_partials=None):
    """Dense-mask form: the top-k residual channels of each unit (as
    resq_select_and_requant) kept at their own positions, the rest zero, and
    that full-width residual requantized.  Returns (sel_idx int32 [U, k],
    m_codes [rows, K/2], m_scales [rows, K/16], m_global fp32 [U])."""
    lib = load()
    _require_cuda(x, codes, scales, g, unit_offsets, row_index, tile_partials)
    x_rows, kk = x.shape
    dev = x.device
    if tile_partials is not None:
        n_units = (x_rows + 127) // 128
        rows_total = x_rows
    else:
        n_units = unit_offsets.numel() - 1
        if rows_total is None:
            raise ValueError("rows_total (host int) is required with unit_offsets")
    sel = torch.empty(n_units, k, dtype=torch.int32, device=dev)
    mc = torch.empty(rows_total, kk // 2, dtype=torch.uint8, device=dev)
    ms = torch.empty(rows_total, kk // 16, dtype=torch.uint8, device=dev)
    mg = torch.empty(n_units, dtype=torch.float32, device=dev)
    ws = _workspace(lib.resq_select_and_requant_workspace_size(kk, rows_total, n_units, k), dev)
    _check(lib.resq_mask_select_and_requant(
        _ptr(x), _dtype_code(x), x_rows, kk, x.stride(0), _ptr(row_index), _ptr(codes),
        _ptr(scales), _ptr(g), _ptr(unit_offsets), n_units, rows_total, k, _ptr(tile_partials),
        _ptr(sel), _ptr(mc), _ptr(ms), _ptr(mg), _ptr(ws), ws.numel(), _stream()),
        "resq_mask_select_and_requant")
    return sel, mc, ms, mg


def moe_w4a4_masked_comp_gemm(m_codes, m_scales, m_global, group_offsets, rows_total,
                              w_codes, w_scales, w_global, out):
    """out [rows_total, N] fp32 += Q(R * M) Q(W)^T per group (the dense-mask
    compensation term); out already holds the main product.  Returns out."""
    lib = load()
    _require_cuda(m_codes, m_scales, m_global, group_offsets, w_codes, w_scales, w_global, out)
    n_exp, n, k_half = w_codes.shape
    if out.dtype != torch.float32 or out.dim() != 2 or out.shape[0] < rows_total \
            or out.shape[1] < n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [rows_total, >= N] with unit column stride")
    _check(lib.moe_w4a4_masked_comp_gemm(
        _ptr(m_codes), _ptr(m_scales), _ptr(m_global), _ptr(group_offsets), n_exp, rows_total,
        k_half * 2, _ptr(w_codes), _ptr(w_scales), _ptr(w_global), n, _ptr(out), out.stride(0),
        _stream()), "moe_w4a4_masked_comp_gemm")
    return out


def moe_w4a4_grouped_gemm(a_codes, a_scales, a_global, group_offsets, rows_total,
                          w_codes, w_scales, w_global, epilogue=EPI_F32, a_row_index=None,
                          sel_idx=None, r_codes=None, r_scales=None, r_global=None,
                          row_weight=None, scatter_index=None, out=None, out_rows=None,
                          out_amax=None):
    """Grouped W4A4 GEMM with the fused compensation term.

    w_codes [E, N, K/2].  Returns out: fp32 [rows_total, N] (EPI_F32), bf16
    [rows_total, N/2] (EPI_SWIGLU_BF16), or the given fp32 out
    [out_rows, N] after the scatter-add (EPI_SCATTER_ADD_F32: out += the
    routed rows; EPI_SCATTER_F32: out = them, allocated when out is None)."""
    lib = load()
    _require_cuda(a_codes, a_scales, a_global, group_offsets, w_codes, w_scales, w_global,
                  a_row_index, sel_idx, r_codes, r_scales, r_global, row_weight, scatter_index,
                  out, out_amax)
    n_exp, n, k_half = w_codes.shape
    kk = k_half * 2
    dev = w_codes.device
    if out is None:
        if epilogue == EPI_F32:
            out = torch.empty(rows_total, n, dtype=torch.float32, device=dev)
        elif epilogue == EPI_SWIGLU_BF16:
            out = torch.empty(rows_total, n // 2, dtype=torch.bfloat16, device=dev)
        elif epilogue == EPI_SCATTER_F32 and out_rows is not None:
            out = torch.empty(out_rows, n, dtype=torch.float32, device=dev)
        else:
            raise ValueError("EPI_SCATTER_ADD_F32 needs an initialised out tensor "
                             "(EPI_SCATTER_F32 an out tensor or out_rows)")
    if out_rows is None:
        out_rows = out.shape[0]
    kc = 0 if sel_idx is None else sel_idx.shape[1]
    ws = _workspace(lib.moe_w4a4_grouped_gemm_workspace_size(n_exp, rows_total, n, kk, epilogue,
                                                             out_rows), dev)
    a_rows = a_codes.shape[0] if a_codes is not None else 0
    _check(lib.moe_w4a4_grouped_gemm(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_global), _ptr(a_row_index), a_rows,
        _ptr(group_offsets), n_exp, rows_total, kk, _ptr(w_codes), _ptr(w_scales),
        _ptr(w_global), n, _ptr(sel_idx), _ptr(r_codes), _ptr(r_scales), _ptr(r_global), kc,
        epilogue, _ptr(row_weight), _ptr(scatter_index), out_rows, _ptr(out), out.stride(0),
        _ptr(out_amax), _ptr(ws), ws.numel(), _stream()), "moe_w4a4_grouped_gemm")
    return out


def qdq_weights(w, want_codes=True):
    """Weight QDQ of w bf16 [nmat, N, K].  Returns (w_qdq bf16, codes, scales, g)."""
    lib = load()
    _require_cuda(w)
    nmat, n, kk = w.shape
    dev = w.device
    w_qdq = torch.empty_like(w)
    codes = torch.empty(nmat, n, kk // 2, dtype=torch.uint8, device=dev) if want_codes else None
    scales = torch.empty(nmat, n, kk // 16, dtype=torch.uint8, device=dev) if want_codes else None
    g = torch.empty(nmat, dtype=torch.float32, device=dev)
    ws = _workspace(lib.qdq_weights_workspace_size(nmat, n, kk), dev)
    _check(lib.qdq_weights(_ptr(w), nmat, n, kk, _ptr(w_qdq), _ptr(codes), _ptr(scales), _ptr(g),
                           _ptr(ws), ws.numel(), _stream()), "qdq_weights")
    return w_qdq, codes, scales, g


def guided_round(x_train, roll_codes, roll_scales, roll_global, want_fq=True, want_hist=True):
    """Rollout-guided rounding.  Returns (codes [M, K/2], x_fq bf16 or None,
    dist_hist int64 [3] or None)."""
    lib = load()
    _require_cuda(x_train, roll_codes, roll_scales, roll_global)
    m, kk = x_train.shape
    dev = x_train.device
    codes = torch.empty(m, kk // 2, dtype=torch.uint8, device=dev)
    fq = torch.empty(m, kk, dtype=torch.bfloat16, device=dev) if want_fq else None
    hist = torch.empty(3, dtype=torch.int64, device=dev) if want_hist else None
    _check(lib.guided_round(_ptr(x_train), _dtype_code(x_train), m, kk, x_train.stride(0),
                            _ptr(roll_codes), _ptr(roll_scales), _ptr(roll_global), _ptr(codes),
                            _ptr(fq), _ptr(hist), _stream()), "guided_round")
    return codes, fq, hist


def mxfp4_qdq_weights(w, want_codes=True):
    """MXFP4 weight QDQ of w bf16 [nmat, N, K] (K % 32 == 0).  Returns (w_qdq
    bf16, codes [nmat, N, K/2] or None, scales [nmat, N, K/32] or None)."""
    lib = load()
    _require_cuda(w)
    nmat, n, kk = w.shape
    dev = w.device
    w_qdq = torch.empty_like(w)
    codes = torch.empty(nmat, n, kk // 2, dtype=torch.uint8, device=dev) if want_codes else None
    scales = torch.empty(nmat, n, kk // 32, dtype=torch.uint8, device=dev) if want_codes else None
    _check(lib.mxfp4_qdq_weights(_ptr(w), nmat, n, kk, _ptr(w_qdq), _ptr(codes), _ptr(scales),
                                 _stream()), "mxfp4_qdq_weights")
    return w_qdq, codes, scales


def mxfp4_guided_round(x_train, roll_codes, roll_scales, want_fq=True, want_hist=True):
    """Rollout-guided rounding against MXFP4 rollout codes [M, K/2] and E8M0
    scales [M, K/32].  Returns (codes, x_fq bf16 or None, dist_hist or None)."""
    lib = load()
    _require_cuda(x_train, roll_codes, roll_scales)
    m, kk = x_train.shape
    dev = x_train.device
    codes = torch.empty(m, kk // 2, dtype=torch.uint8, device=dev)
    fq = torch.empty(m, kk, dtype=torch.bfloat16, device=dev) if want_fq else None
    hist = torch.empty(3, dtype=torch.int64, device=dev) if want_hist else None
    _check(lib.mxfp4_guided_round(_ptr(x_train), _dtype_code(x_train), m, kk, x_train.stride(0),
                                  _ptr(roll_codes), _ptr(roll_scales), _ptr(codes), _ptr(fq),
                                  _ptr(hist), _stream()), "mxfp4_guided_round")
    return codes, fq, hist


def mxfp4_guided_round_record(x_train, record, roll_scales, want_fq=True, want_moved=True):
    """Guided rounding from the mantissa-only record [M, K/8] of MXFP4 rollout
    codes, with their E8M0 scales [M, K/32].  Returns (codes [M, K/2], x_fq
    bf16 or None, moved int64 [2] or None)."""
    lib = load()
    _require_cuda(x_train, record, roll_scales)
    m, kk = x_train.shape
    dev = x_train.device
    codes = torch.empty(m, kk // 2, dtype=torch.uint8, device=dev)
    fq = torch.empty(m, kk, dtype=torch.bfloat16, device=dev) if want_fq else None
    moved = torch.empty(2, dtype=torch.int64, device=dev) if want_moved else None
    _check(lib.mxfp4_guided_round_record(_ptr(x_train), _dtype_code(x_train), m, kk,
                                         x_train.stride(0), _ptr(record), _ptr(roll_scales),
                                         _ptr(codes), _ptr(fq), _ptr(moved), _stream()),
           "mxfp4_guided_round_record")
    return codes, fq, moved


def guidance_record_pack(roll_codes):
    """Mantissa-only guidance record of rollout codes [M, K/2]: returns [M, K/8]."""
    lib = load()
    _require_cuda(roll_codes)
    m, kh = roll_codes.shape
    record = torch.empty(m, kh // 4, dtype=torch.uint8, device=roll_codes.device)
    _check(lib.guidance_record_pack(_ptr(roll_codes), m, kh * 2, _ptr(record), _stream()),
           "guidance_record_pack")
    return record


def guided_round_record(x_train, record, roll_scales, roll_global, want_fq=True, want_moved=True):
    """Rollout-guided rounding from the mantissa-only record.  Returns (codes
    [M, K/2], x_fq bf16 or None, moved int64 [2] or None)."""
    lib = load()
    _require_cuda(x_train, record, roll_scales, roll_global)
    m, kk = x_train.shape
    dev = x_train.device
    codes = torch.empty(m, kk // 2, dtype=torch.uint8, device=dev)
    fq = torch.empty(m, kk, dtype=torch.bfloat16, device=dev) if want_fq else None
    moved = torch.empty(2, dtype=torch.int64, device=dev) if want_moved else None
    _check(lib.guided_round_record(_ptr(x_train), _dtype_code(x_train), m, kk, x_train.stride(0),
                                   _ptr(record), _ptr(roll_scales), _ptr(roll_global), _ptr(codes),
                                   _ptr(fq), _ptr(moved), _stream()), "guided_round_record")
    return codes, fq, moved


# ---------------------------------------------------------------------------
# MXFP4 variant
# ---------------------------------------------------------------------------
def mxfp4_quantize(x, tile_partials=False):
    """MXFP4 quantization of x [M, K] (bf16/fp32, GPU).

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32] (E8M0),
    tile_partials fp32 [ceil(M/128), K] or None)."""
    lib = load()
    _require_cuda(x)
    m, k = x.shape
    dev = x.device
    codes = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(m, k // 32, dtype=torch.uint8, device=dev)
    tp = torch.empty((m + 127) // 128, k, dtype=torch.float32, device=dev) if tile_partials else None
    _check(lib.mxfp4_quantize(_ptr(x), _dtype_code(x), m, k, x.stride(0), _ptr(codes),
                              _ptr(scales), _ptr(tp), _stream()), "mxfp4_quantize")
    return codes, scales, tp


def mxfp4_resq_select_and_requant(x, codes, scales, k, unit_offsets=None, rows_total=None,
                                  row_index=None, tile_partials=None):
    """MXFP4 residual selection and requantization (see resq_select_and_requant).
    Returns (sel_idx int32 [U, k], r_codes [rows, k/2], r_scales [rows, k/32])."""
    lib = load()
    _require_cuda(x, codes, scales, unit_offsets, row_index, tile_partials)
    x_rows, kk = x.shape
    dev = x.device
    if tile_partials is not None:
        n_units = (x_rows + 127) // 128
        rows_total = x_rows
    else:
        n_units = unit_offsets.numel() - 1
        if rows_total is None:
            raise ValueError("rows_total (host int) is required with unit_offsets")
    sel = torch.empty(n_units, k, dtype=torch.int32, device=dev)
    rc = torch.empty(rows_total, k // 2, dtype=torch.uint8, device=dev)
    rs = torch.empty(rows_total, k // 32, dtype=torch.uint8, device=dev)
    ws = _workspace(lib.mxfp4_resq_select_and_requant_workspace_size(kk, rows_total, n_units, k), dev)
    _check(lib.mxfp4_resq_select_and_requant(
        _ptr(x), _dtype_code(x), x_rows, kk, x.stride(0), _ptr(row_index), _ptr(codes),
        _ptr(scales), _ptr(unit_offsets), n_units, rows_total, k, _ptr(tile_partials),
        _ptr(sel), _ptr(rc), _ptr(rs), _ptr(ws), ws.numel(), _stream()),
        "mxfp4_resq_select_and_requant")
    return sel, rc, rs


def moe_mxfp4_grouped_gemm(a_codes, a_scales, group_offsets, rows_total, w_codes, w_scales,
                           epilogue=EPI_F32, a_row_index=None, sel_idx=None, r_codes=None,
                           r_scales=None, row_weight=None, scatter_index=None, out=None,
                           out_rows=None, out_amax=None):
    """Grouped MXFP4 W4A4 GEMM with the fused compensation term (outputs as
    moe_w4a4_grouped_gemm)."""
    lib = load()
    _require_cuda(a_codes, a_scales, group_offsets, w_codes, w_scales, a_row_index, sel_idx,
                  r_codes, r_scales, row_weight, scatter_index, out, out_amax)
    n_exp, n, k_half = w_codes.shape
    kk = k_half * 2
    dev = w_codes.device
    if out is None:
        if epilogue == EPI_F32:
            out = torch.empty(rows_total, n, dtype=torch.float32, device=dev)
        elif epilogue == EPI_SWIGLU_BF16:
            out = torch.empty(rows_total, n // 2, dtype=torch.bfloat16, device=dev)
        elif epilogue == EPI_SCATTER_F32 and out_rows is not None:
            out = torch.empty(out_rows, n, dtype=torch.float32, device=dev)
        else:
            raise ValueError("EPI_SCATTER_ADD_F32 needs an initialised out tensor "
                             "(EPI_SCATTER_F32 an out tensor or out_rows)")
    if out_rows is None:
        out_rows = out.shape[0]
    kc = 0 if sel_idx is None else sel_idx.shape[1]
    ws = _workspace(lib.moe_mxfp4_grouped_gemm_workspace_size(n_exp, rows_total, n, kk, epilogue,
                                                              out_rows), dev)
    a_rows = a_codes.shape[0] if a_codes is not None else 0
    _check(lib.moe_mxfp4_grouped_gemm(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_row_index), a_rows, _ptr(group_offsets), n_exp,
        rows_total, kk, _ptr(w_codes), _ptr(w_scales), n, _ptr(sel_idx), _ptr(r_codes),
        _ptr(r_scales), kc, epilogue, _ptr(row_weight), _ptr(scatter_index), out_rows, _ptr(out),
        out.stride(0), _ptr(out_amax), _ptr(ws), ws.numel(), _stream()), "moe_mxfp4_grouped_gemm")
    return out


def mxfp8_quantize(x):
    """MXFP8 quantization of activations x [M, K] (bf16/fp32, GPU).
    Returns (codes uint8 [M, K] E4M3 bytes, scales uint8 [M, K/32] E8M0)."""
    lib = load()
    _require_cuda(x)
    m, k = x.shape
    codes = torch.empty(m, k, dtype=torch.uint8, device=x.device)
    scales = torch.empty(m, k // 32, dtype=torch.uint8, device=x.device)
    _check(lib.mxfp8_quantize(_ptr(x), _dtype_code(x), m, k, x.stride(0), _ptr(codes), _ptr(scales),
                              _stream()), "mxfp8_quantize")
    return codes, scales


def moe_mxfp4_w4a8_grouped_gemm(a_codes, a_scales, group_offsets, rows_total, w_codes, w_scales,
                                epilogue=EPI_F32, a_row_index=None, row_weight=None,
                                scatter_index=None, out=None, out_rows=None, out_amax=None):
    """Grouped W4A8 GEMM: MXFP8 activations [rows, K] x MXFP4 weights [E, N, K/2]
    (outputs as moe_w4a4_grouped_gemm)."""
    lib = load()
    _require_cuda(a_codes, a_scales, group_offsets, w_codes, w_scales, a_row_index, row_weight,
                  scatter_index, out, out_amax)
    n_exp, n, k_half = w_codes.shape
    kk = k_half * 2
    dev = w_codes.device
    if out is None:
        if epilogue == EPI_F32:
            out = torch.empty(rows_total, n, dtype=torch.float32, device=dev)
        elif epilogue == EPI_SWIGLU_BF16:
            out = torch.empty(rows_total, n // 2, dtype=torch.bfloat16, device=dev)
        elif epilogue == EPI_SCATTER_F32 and out_rows is not None:
            out = torch.empty(out_rows, n, dtype=torch.float32, device=dev)
        else:
            raise ValueError("EPI_SCATTER_ADD_F32 needs an initialised out tensor "
                             "(EPI_SCATTER_F32 an out tensor or out_rows)")
    if out_rows is None:
        out_rows = out.shape[0]
    ws = _workspace(lib.moe_mxfp4_w4a8_grouped_gemm_workspace_size(n_exp, rows_total, n, kk,
                                                                   epilogue, out_rows), dev)
    a_rows = a_codes.shape[0] if a_codes is not None else 0
    _check(lib.moe_mxfp4_w4a8_grouped_gemm(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_row_index), a_rows, _ptr(group_offsets), n_exp,
        rows_total, kk, _ptr(w_codes), _ptr(w_scales), n, epilogue, _ptr(row_weight),
        _ptr(scatter_index), out_rows, _ptr(out), out.stride(0), _ptr(out_amax), _ptr(ws),
        ws.numel(), _stream()), "moe_mxfp4_w4a8_grouped_gemm")
    return out
