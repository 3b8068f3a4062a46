"""Thin Python binding of the C ABI (include/mxfp8moe.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch when the caller does not pass them, and every step of
the computation runs in the HIP kernels of libmxfp8moe.so on the current
torch stream (or the stream given).  The entry points have the C names
without the ``mxfp8_`` prefix.
"""

from dataclasses import dataclass
from typing import Optional

import torch

from . import _native

ROWWISE = 1
COLWISE = 2
LAYOUT_NT, LAYOUT_NN, LAYOUT_TN = 0, 1, 2
_LAYOUTS = {"NT": LAYOUT_NT, "NN": LAYOUT_NN, "TN": LAYOUT_TN, 0: 0, 1: 1, 2: 2}
_OUT = {torch.float32: 0, torch.bfloat16: 1}


@dataclass
class MXFP8Tensor:
    """Row-wise and/or column-wise MXFP8 copies of a [T, K] tensor.

    row_data [T, K] u8 + row_scale [T, K/32] u8; col_data [K, T] u8 +
    col_scale [K, T/32] u8 (the column-wise copy stored transposed).
    """
    row_data: Optional[torch.Tensor] = None
    row_scale: Optional[torch.Tensor] = None
    col_data: Optional[torch.Tensor] = None
    col_scale: Optional[torch.Tensor] = None


def _lib():
    return _native.load()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, dtype, shape, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _as_shape(t, shape, name):
    """View a contiguous u8 operand with the expected number of bytes as `shape`."""
    n = 1
    for d in shape:
        n *= d
    if t.numel() != n:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    t = t.view(shape)
    _need(t, torch.uint8, shape, name)
    return t


def _splits(m_splits, name="m_splits"):
    if not isinstance(m_splits, torch.Tensor) or not m_splits.is_cuda or m_splits.dtype != torch.int64:
        raise ValueError(f"{name} must be a device int64 tensor")
    if not m_splits.is_contiguous() or m_splits.dim() != 1:
        raise ValueError(f"{name} must be a contiguous 1-D tensor")
    return m_splits


def _mx_outputs(out, usage, t, k, like):
    """Allocate (or check) the requested row-/column-wise buffers of a [t, k] tensor."""
    out = out or MXFP8Tensor()
    if usage & ROWWISE:
        if out.row_data is None:
            out.row_data = _empty((t, k), torch.uint8, like)
            out.row_scale = _empty((t, k // 32), torch.uint8, like)
        _need(out.row_data, torch.uint8, (t, k), "row_data")
        _need(out.row_scale, torch.uint8, (t, k // 32), "row_scale")
    if usage & COLWISE:
        if out.col_data is None:
            out.col_data = _empty((k, t), torch.uint8, like)
            out.col_scale = _empty((k, t // 32), torch.uint8, like)
        _need(out.col_data, torch.uint8, (k, t), "col_data")
        _need(out.col_scale, torch.uint8, (k, t // 32), "col_scale")
    return out


def _mx_ptrs(out, usage):
    row = usage & ROWWISE
    col = usage & COLWISE
    return (_ptr(out.row_data) if row else None, _ptr(out.row_scale) if row else None,
            _ptr(out.col_data) if col else None, _ptr(out.col_scale) if col else None)


def group_quantize(x, usage=ROWWISE, out: Optional[MXFP8Tensor] = None, noop_flag=None,
                   stream=None):
    """bf16 [T, K] (or [G, N, K], taken as [G*N, K]) -> MXFP8Tensor.

    noop_flag: optional device int32 [1]; when it holds a non-zero value as
    the kernels run, nothing is written and `out` keeps its contents.
    """
    lib = _lib()
    if x.dim() != 2:
        x = x.reshape(-1, x.shape[-1])
    t, k = x.shape
    _need(x, torch.bfloat16, (t, k), "x")
    out = _mx_outputs(out, usage, t, k, x)
    if noop_flag is not None:
        _need(noop_flag, torch.int32, (1,), "noop_flag")
    st = lib.mxfp8_group_quantize(_ptr(x), t, k, usage, *_mx_ptrs(out, usage), _ptr(noop_flag),
                                  _stream(stream))
    _native.check(st, "mxfp8_group_quantize")
    return out


def swiglu_quantize(h, usage=ROWWISE | COLWISE, out: Optional[MXFP8Tensor] = None,
                    stream=None):
    """h [T, 2F] bf16 -> MXFP8Tensor of a = silu(h[:, :F]) * h[:, F:] (bf16
    rounded, as swiglu_fwd gives it) without writing a."""
    lib = _lib()
    t, f2 = h.shape
    f = f2 // 2
    _need(h, torch.bfloat16, (t, 2 * f), "h")
    out = _mx_outputs(out, usage, t, f, h)
    st = lib.mxfp8_swiglu_quantize(_ptr(h), t, f, usage, *_mx_ptrs(out, usage), _stream(stream))
    _native.check(st, "mxfp8_swiglu_quantize")
    return out


def dbias_workspace_bytes(t, n):
    return int(_lib().mxfp8_dbias_workspace_bytes(t, n))


def _workspace(t, n, like, workspace):
    need = dbias_workspace_bytes(t, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device buffer of at least {need} bytes")
    return workspace


def requant_colwise(row_data, row_scale, m_splits=None, with_dbias=False, out=None,
                    dbias=None, workspace=None, stream=None):
    """Row-wise MXFP8 [T, K] -> column-wise copy ([K, T], [K, T/32]) (+ dbias [G, K])."""
    lib = _lib()
    t, k = row_data.shape
    _need(row_data, torch.uint8, (t, k), "row_data")
    _need(row_scale, torch.uint8, (t, k // 32), "row_scale")
    out = out or MXFP8Tensor(row_data=row_data, row_scale=row_scale)
    if out.col_data is None:
        out.col_data = _empty((k, t), torch.uint8, row_data)
        out.col_scale = _empty((k, t // 32), torch.uint8, row_data)
    _need(out.col_data, torch.uint8, (k, t), "col_data")
    _need(out.col_scale, torch.uint8, (k, t // 32), "col_scale")
    g = 0
    ms = None
    if with_dbias:
        ms = _splits(m_splits)
        g = ms.numel()
        if dbias is None:
            dbias = _empty((g, k), torch.float32, row_data)
        _need(dbias, torch.float32, (g, k), "dbias")
        workspace = _workspace(t, k, row_data, workspace)
    st = lib.mxfp8_requant_colwise(
        _ptr(row_data), _ptr(row_scale), t, k, _ptr(out.col_data), _ptr(out.col_scale),
        _ptr(ms), g, _ptr(dbias) if with_dbias else None,
        _ptr(workspace) if with_dbias else None,
        workspace.numel() * workspace.element_size() if with_dbias else 0, _stream(stream))
    _native.check(st, "mxfp8_requant_colwise")
    return (out, dbias) if with_dbias else out


def group_quantize_requant(x, m_splits=None, with_dbias=False, out=None, dbias=None,
                           workspace=None, stream=None):
    """bf16 [T, K] -> MXFP8Tensor with the row-wise copy and the column-wise
    copy requantized from it (+ dbias [G, K] from the dequantized row-wise
    values), in one pass: the bytes of group_quantize(ROWWISE) followed by
    requant_colwise.  Returns the tensor, or (tensor, dbias) with_dbias."""
    lib = _lib()
    t, k = x.shape
    _need(x, torch.bfloat16, (t, k), "x")
    out = _mx_outputs(out, ROWWISE | COLWISE, t, k, x)
    g = 0
    ms = None
    if with_dbias:
        ms = _splits(m_splits)
        g = ms.numel()
        if dbias is None:
            dbias = _empty((g, k), torch.float32, x)
        _need(dbias, torch.float32, (g, k), "dbias")
        workspace = _workspace(t, k, x, workspace)
    st = lib.mxfp8_group_quantize_requant(
        _ptr(x), t, k, _ptr(out.row_data), _ptr(out.row_scale), _ptr(out.col_data),
        _ptr(out.col_scale), _ptr(ms), g, _ptr(dbias) if with_dbias else None,
        _ptr(workspace) if with_dbias else None,
        workspace.numel() * workspace.element_size() if with_dbias else 0, _stream(stream))
    _native.check(st, "mxfp8_group_quantize_requant")
    return (out, dbias) if with_dbias else out


NOALLOC_SCRATCH_BYTES = 32 << 20   # MXFP8_NOALLOC_SCRATCH_BYTES of the C header


def group_quantize_requant_noalloc(x, m_splits=None, with_dbias=False, out=None, dbias=None,
                                   stream=None):
    """group_quantize_requant without a workspace: the dbias partial sums go
    to the library's static per-GPU scratch (mxfp8_group_quantize_requant_
    noalloc; with dbias, (T/128) * K * 4 <= NOALLOC_SCRATCH_BYTES).  Calls
    with dbias that overlap on one GPU race on that scratch.  Pass `out` (and
    `dbias`) to keep the call free of allocations."""
    lib = _lib()
    t, k = x.shape
    _need(x, torch.bfloat16, (t, k), "x")
    out = _mx_outputs(out, ROWWISE | COLWISE, t, k, x)
    g = 0
    ms = None
    if with_dbias:
        ms = _splits(m_splits)
        g = ms.numel()
        if dbias is None:
            dbias = _empty((g, k), torch.float32, x)
        _need(dbias, torch.float32, (g, k), "dbias")
    st = lib.mxfp8_group_quantize_requant_noalloc(
        _ptr(x), t, k, _ptr(out.row_data), _ptr(out.row_scale), _ptr(out.col_data),
        _ptr(out.col_scale), _ptr(ms), g, _ptr(dbias) if with_dbias else None, _stream(stream))
    _native.check(st, "mxfp8_group_quantize_requant_noalloc")
    return (out, dbias) if with_dbias else out


def grouped_dbias(row_data, row_scale, m_splits, dbias=None, workspace=None, stream=None):
    """Row-wise MXFP8 dY [T, N] -> dbias [G, N] fp32 (sum over each expert's rows)."""
    lib = _lib()
    t, n = row_data.shape
    _need(row_data, torch.uint8, (t, n), "row_data")
    _need(row_scale, torch.uint8, (t, n // 32), "row_scale")
    ms = _splits(m_splits)
    g = ms.numel()
    if dbias is None:
        dbias = _empty((g, n), torch.float32, row_data)
    _need(dbias, torch.float32, (g, n), "dbias")
    workspace = _workspace(t, n, row_data, workspace)
    st = lib.mxfp8_grouped_dbias(_ptr(row_data), _ptr(row_scale), t, n, _ptr(ms), g,
                                 _ptr(dbias), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _native.check(st, "mxfp8_grouped_dbias")
    return dbias


def grouped_scaled_bias_grad(row_data, row_scale, m_splits, scales=None, bias=None,
                             want_dbias=True, want_dscales=True, workspace=None, out=None,
                             stream=None):
    """Gradients of a routing-scaled bias from row-wise MXFP8 dY [T, N]:
    dbias [G, N] = sum over each expert's rows of scales[r] dY[r] (needs
    scales [T] fp32) and dscales [T] = dY[r] . bias[g] (needs bias [G, N]
    fp32).  out: optional (dbias, dscales) buffers to write into.  Returns
    (dbias or None, dscales or None)."""
    lib = _lib()
    t, n = row_data.shape
    _need(row_data, torch.uint8, (t, n), "row_data")
    _need(row_scale, torch.uint8, (t, n // 32), "row_scale")
    ms = _splits(m_splits)
    g = ms.numel()
    dbias, dscales = (None, None) if out is None else out
    if want_dbias:
        _need(scales, torch.float32, (t,), "scales")
        dbias = _empty((g, n), torch.float32, row_data) if dbias is None else dbias
        _need(dbias, torch.float32, (g, n), "dbias")
    else:
        dbias = None
    if want_dscales:
        _need(bias, torch.float32, (g, n), "bias")
        dscales = _empty((t,), torch.float32, row_data) if dscales is None else dscales
        _need(dscales, torch.float32, (t,), "dscales")
    else:
        dscales = None
    need = lib.mxfp8_scaled_bias_workspace_bytes(t, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=row_data.device)
    st = lib.mxfp8_grouped_scaled_bias_grad(
        _ptr(row_data), _ptr(row_scale), t, n, _ptr(ms), g, _ptr(scales) if want_dbias else None,
        _ptr(bias) if want_dscales else None, _ptr(dbias), _ptr(dscales), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _native.check(st, "mxfp8_grouped_scaled_bias_grad")
    return dbias, dscales


def gemm_workspace_bytes():
    return int(_lib().mxfp8_grouped_gemm_workspace_bytes())


def _gemm_workspace(workspace):
    need = gemm_workspace_bytes()
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device buffer of at least {need} bytes")
    return workspace


def grouped_gemm(layout, a_data, a_scale, b_data, b_scale, m_splits, tokens, n, k,
                 out_dtype=torch.float32, out=None, stream=None, workspace=None):
    """One grouped GEMM of an expert linear (in_features k, out_features n).

    layout "NT" (forward): a = X row-wise [T, k], b = W row-wise [G, n, k] -> [T, n]
    layout "NN" (dgrad):   a = dY row-wise [T, n], b = W column-wise [k, G*n] -> [T, k]
    layout "TN" (wgrad):   a = dY column-wise [n, T], b = X column-wise [k, T] -> [G, n, k]

    workspace: optional device buffer of gemm_workspace_bytes(); with it the
    wgrad tiles are handed out dynamically (mxfp8_grouped_gemm_ws), same bytes.
    """
    lib = _lib()
    lay = _LAYOUTS[layout]
    ms = _splits(m_splits)
    g = ms.numel()
    t = tokens
    if out_dtype not in _OUT:
        raise NotImplementedError(f"output dtype {out_dtype} is not supported")
    if lay == LAYOUT_NT:
        shapes = ((t, k), (t, k // 32), (g * n, k), (g * n, k // 32), (t, n))
    elif lay == LAYOUT_NN:
        shapes = ((t, n), (t, n // 32), (k, g * n), (k, g * n // 32), (t, k))
    else:
        shapes = ((n, t), (n, t // 32), (k, t), (k, t // 32), (g, n, k))
    a2 = _as_shape(a_data, shapes[0], "a_data")
    as2 = _as_shape(a_scale, shapes[1], "a_scale")
    b2 = _as_shape(b_data, shapes[2], "b_data")
    bs2 = _as_shape(b_scale, shapes[3], "b_scale")
    if out is None:
        out = _empty(shapes[4], out_dtype, a2)
    _need(out, out_dtype, shapes[4], "out")
    if workspace is None:
        st = lib.mxfp8_grouped_gemm(lay, _ptr(a2), _ptr(as2), _ptr(b2), _ptr(bs2), _ptr(out),
                                    _OUT[out_dtype], t, n, k, _ptr(ms), g, _stream(stream))
        _native.check(st, "mxfp8_grouped_gemm")
    else:
        ws = _gemm_workspace(workspace)
        st = lib.mxfp8_grouped_gemm_ws(lay, _ptr(a2), _ptr(as2), _ptr(b2), _ptr(bs2), _ptr(out),
                                       _OUT[out_dtype], t, n, k, _ptr(ms), g, _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream))
        _native.check(st, "mxfp8_grouped_gemm_ws")
    return out


def grouped_gemm_swiglu_quantize(a_data, a_scale, b_data, b_scale, m_splits, tokens, f, k,
                                 usage=ROWWISE | COLWISE, h=None, out=None, stream=None):
    """Forward of the fused MLP's FC1 with SwiGLU + quantize in the epilogue:
    h [T, 2F] = X W1_g^T (bf16; a = X row-wise [T, k], b = W1 row-wise
    [G, 2F, k]) and the MXFP8Tensor of a = silu(h[:, :F]) * h[:, F:] (the
    bytes of grouped_gemm + swiglu_quantize).  Returns (h, MXFP8Tensor)."""
    lib = _lib()
    ms = _splits(m_splits)
    g = ms.numel()
    t = tokens
    a2 = _as_shape(a_data, (t, k), "a_data")
    as2 = _as_shape(a_scale, (t, k // 32), "a_scale")
    b2 = _as_shape(b_data, (g * 2 * f, k), "b_data")
    bs2 = _as_shape(b_scale, (g * 2 * f, k // 32), "b_scale")
    if h is None:
        h = _empty((t, 2 * f), torch.bfloat16, a2)
    _need(h, torch.bfloat16, (t, 2 * f), "h")
    out = _mx_outputs(out, usage, t, f, a2)
    st = lib.mxfp8_grouped_gemm_swiglu_quantize(
        _ptr(a2), _ptr(as2), _ptr(b2), _ptr(bs2), _ptr(h), t, f, k, _ptr(ms), g, usage,
        *_mx_ptrs(out, usage), _stream(stream))
    _native.check(st, "mxfp8_grouped_gemm_swiglu_quantize")
    return h, out


def grouped_gemm_wgrad_accumulate(a_data, a_scale, b_data, b_scale, m_splits, tokens, n, k,
                                  main_grad, stream=None, workspace=None):
    """wgrad added into an fp32 main_grad [G, n, k] in place:
    main_grad[g] += dY_g^T X_g (a = dY column-wise [n, T], b = X column-wise
    [k, T]); experts without tokens keep their main_grad untouched."""
    lib = _lib()
    ms = _splits(m_splits)
    g = ms.numel()
    t = tokens
    a2 = _as_shape(a_data, (n, t), "a_data")
    as2 = _as_shape(a_scale, (n, t // 32), "a_scale")
    b2 = _as_shape(b_data, (k, t), "b_data")
    bs2 = _as_shape(b_scale, (k, t // 32), "b_scale")
    _need(main_grad, torch.float32, (g, n, k), "main_grad")
    if workspace is None:
        st = lib.mxfp8_grouped_gemm_wgrad_accumulate(_ptr(a2), _ptr(as2), _ptr(b2), _ptr(bs2),
                                                     _ptr(main_grad), t, n, k, _ptr(ms), g,
                                                     _stream(stream))
        _native.check(st, "mxfp8_grouped_gemm_wgrad_accumulate")
    else:
        ws = _gemm_workspace(workspace)
        st = lib.mxfp8_grouped_gemm_wgrad_accumulate_ws(
            _ptr(a2), _ptr(as2), _ptr(b2), _ptr(bs2), _ptr(main_grad), t, n, k, _ptr(ms), g,
            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
        _native.check(st, "mxfp8_grouped_gemm_wgrad_accumulate_ws")
    return main_grad


def validate_splits(m_splits, tokens, flag=None, stream=None):
    """Enqueue the device-side split check; returns the device int32 flag tensor."""
    lib = _lib()
    ms = _splits(m_splits)
    if flag is None:
        flag = _empty((1,), torch.int32, ms)
    st = lib.mxfp8_validate_splits(_ptr(ms), ms.numel(), tokens, _ptr(flag), _stream(stream))
    _native.check(st, "mxfp8_validate_splits")
    return flag


def swiglu_fwd(h, out=None, stream=None):
    """h [T, 2F] bf16 -> silu(h[:, :F]) * h[:, F:] as bf16 [T, F]."""
    lib = _lib()
    t, f2 = h.shape
    f = f2 // 2
    _need(h, torch.bfloat16, (t, 2 * f), "h")
    if out is None:
        out = _empty((t, f), torch.bfloat16, h)
    _need(out, torch.bfloat16, (t, f), "out")
    _native.check(lib.mxfp8_swiglu_fwd(_ptr(h), t, f, _ptr(out), _stream(stream)),
                  "mxfp8_swiglu_fwd")
    return out


def swiglu_bwd_quantize(h, da, m_splits=None, with_dbias=False, out=None, dbias=None,
                        workspace=None, stream=None):
    """SwiGLU backward of h [T, 2F] and da [T, F] (bf16) quantized as
    group_quantize_requant quantizes dh [T, 2F], without writing dh: the bytes
    (and dbias [G, 2F]) of swiglu_bwd followed by group_quantize_requant.
    Returns the tensor, or (tensor, dbias) with_dbias."""
    lib = _lib()
    t, k = h.shape
    f = k // 2
    _need(h, torch.bfloat16, (t, 2 * f), "h")
    _need(da, torch.bfloat16, (t, f), "da")
    out = _mx_outputs(out, ROWWISE | COLWISE, t, k, h)
    g = 0
    ms = None
    if with_dbias:
        ms = _splits(m_splits)
        g = ms.numel()
        if dbias is None:
            dbias = _empty((g, k), torch.float32, h)
        _need(dbias, torch.float32, (g, k), "dbias")
        workspace = _workspace(t, k, h, workspace)
    st = lib.mxfp8_swiglu_bwd_quantize(
        _ptr(h), _ptr(da), t, f, _ptr(out.row_data), _ptr(out.row_scale), _ptr(out.col_data),
        _ptr(out.col_scale), _ptr(ms), g, _ptr(dbias) if with_dbias else None,
        _ptr(workspace) if with_dbias else None,
        workspace.numel() * workspace.element_size() if with_dbias else 0, _stream(stream))
    _native.check(st, "mxfp8_swiglu_bwd_quantize")
    return (out, dbias) if with_dbias else out


def swiglu_bwd(h, da, out=None, stream=None):
    """Gradient of swiglu_fwd w.r.t. h, given da [T, F]; returns bf16 [T, 2F]."""
    lib = _lib()
    t, f2 = h.shape
    f = f2 // 2
    _need(h, torch.bfloat16, (t, 2 * f), "h")
    _need(da, torch.bfloat16, (t, f), "da")
    if out is None:
        out = _empty((t, 2 * f), torch.bfloat16, h)
    _need(out, torch.bfloat16, (t, 2 * f), "out")
    _native.check(lib.mxfp8_swiglu_bwd(_ptr(h), _ptr(da), t, f, _ptr(out), _stream(stream)),
                  "mxfp8_swiglu_bwd")
    return out


def convert_sweep(mode, stream=None):
    """Diagnostic: the device conversion helpers over every (value, scale byte)
    pair (layouts in mxfp8_convert_sweep's header comment); a uint8 tensor."""
    lib = _lib()
    need = lib.mxfp8_convert_sweep_bytes(mode)
    if need == 0:
        raise ValueError(f"unknown sweep mode {mode}")
    out = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = lib.mxfp8_convert_sweep(mode, _ptr(out), need, _stream(stream))
    _native.check(st, "mxfp8_convert_sweep")
    return out
