"""Cactus Quants (CQ) matrix products on one AMD Instinct MI355X (gfx950).

Thin Python binding of ``libcq.so``, the C-ABI library declared in
``include/cq.h``.  This module only marshals arguments: it checks tensor
metadata, passes raw device pointers and the current HIP stream, and turns
status codes into exceptions.  Every step of the computation runs in the HIP
kernels of the library; PyTorch supplies device memory and streams.

The library must be built first (``python hadamard_rotated_codebook_amd/build.py``);
importing this package without it raises ``ImportError`` -- there is no
fallback path.

Functions carry the C names: ``cq_blob_bytes``, ``cq_workspace_bytes``,
``cq_rotate_acts``, ``cq_matvec``, ``cq_rotate_matvec``, ``cq_rotate_matvec_noalloc``,
``cq_rotate_multi_matvec``, ``cq_rotate_multi_workspace_bytes``,
``cq_quantize_acts_int8``, ``cq_matvec_w2a8_quantized``, ``cq_matvec_w2a8``,
``cq_gather_rows``, ``cq_gemm``, ``cq_quantize``.
"""
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LIB_PATH", "CQError", "CQMatrix", "CQ_GROUP", "CQ_MAX_MATVEC_BATCH", "workspace_for",
    "cq_version", "cq_blob_bytes", "cq_workspace_bytes",
    "cq_rotate_acts", "cq_matvec", "cq_rotate_matvec", "cq_rotate_matvec_noalloc", "cq_rotate_multi_matvec",
    "cq_rotate_multi_workspace_bytes", "cq_quantize_acts_int8", "cq_matvec_w2a8_quantized", "cq_matvec_w2a8",
    "cq_gather_rows", "cq_gemm", "cq_quantize", "cq_quantize_rows", "cq_kv_scores_workspace_bytes",
    "cq_kv_scores", "cq_matvec_t", "cq_kv_append", "cq_kv_attention", "cq_read_probe",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run: python hadamard_rotated_codebook_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

CQ_GROUP = 128
CQ_MAX_MATVEC_BATCH = 8
_F32, _F16, _BF16 = 0, 1, 2
_DTYPES = {torch.float32: _F32, torch.float16: _F16, torch.bfloat16: _BF16}
OP_MATVEC, OP_GEMM, OP_ROTATE_MATVEC, OP_W2A8, OP_MATVEC_T = 0, 1, 2, 3, 4


class _Matrix(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("blob", ctypes.c_void_p), ("blob_bytes", ctypes.c_uint64),
        ("levels", ctypes.POINTER(ctypes.c_float)),
    ]


_i32, _i64, _u64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
_MP = ctypes.POINTER(_Matrix)
_SIGS = {
    "cq_version": (_i32, []),
    "cq_status_string": (ctypes.c_char_p, [_i32]),
    "cq_blob_bytes": (_i32, [_i32, _i32, _i64, _i64, ctypes.POINTER(_u64)]),
    "cq_workspace_bytes": (_i32, [_i32, _MP, _i64, ctypes.POINTER(_u64)]),
    "cq_rotate_acts": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _vp]),
    "cq_matvec": (_i32, [_MP, _vp, _i64, _vp, _vp, _u64, _vp]),
    "cq_rotate_matvec": (_i32, [_MP, _vp, _i64, _vp, _vp, _u64, _vp]),
    "cq_rotate_matvec_noalloc": (_i32, [_MP, _vp, _i64, _vp, _vp]),
    "cq_rotate_multi_matvec": (_i32, [_MP, _i32, _vp, _i64, ctypes.POINTER(_vp), _vp, _u64, _vp]),
    "cq_rotate_multi_workspace_bytes": (_i32, [_MP, _i32, _i64, ctypes.POINTER(_u64)]),
    "cq_quantize_acts_int8": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "cq_matvec_w2a8_quantized": (_i32, [_MP, _vp, _vp, _i64, _vp, _vp]),
    "cq_matvec_w2a8": (_i32, [_MP, _vp, _i64, _vp, _vp, _u64, _vp]),
    "cq_gather_rows": (_i32, [_MP, _vp, _i64, _vp, _i32, _vp]),
    "cq_gemm": (_i32, [_MP, _vp, _i64, _vp, _vp, _u64, _vp]),
    "cq_quantize": (_i32, [_vp, _i64, _i64, _i32, _i32, ctypes.POINTER(ctypes.c_float), _vp, _u64, _vp]),
    "cq_quantize_rows": (_i32, [_vp, _i64, _MP, _i64, _vp]),
    "cq_kv_scores_workspace_bytes": (_i32, [_MP, _i32, _i32, _i32, ctypes.POINTER(_u64)]),
    "cq_kv_scores": (_i32, [_MP, _vp, _i32, _i32, _i32, _vp, _vp, _u64, _vp]),
    "cq_kv_attention": (_i32, [_MP, _MP, _i64, _vp, _i32, _i32, _i32, ctypes.c_float, _vp, _vp]),
    "cq_kv_append": (_i32, [_MP, _MP, _vp, _vp, _i64, _i64, _vp]),
    "cq_matvec_t": (_i32, [_MP, _vp, _i64, _vp, _vp, _u64, _vp]),
    "cq_read_probe": (_i32, [_vp, _u64, _vp, _u64, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class CQError(RuntimeError):
    """A libcq call returned a non-zero cq_status."""

    def __init__(self, status):
        self.status = int(status)
        super().__init__(f"cq_status {self.status}: {_lib.cq_status_string(self.status).decode()}")


def _check(status):
    if status != 0:
        raise CQError(status)


def _stream():
    # the current device's current stream as a raw handle (building a
    # torch.cuda.Stream object per call costs several microseconds)
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def _levels_array(levels):
    if levels is None:
        return None, None
    arr = np.ascontiguousarray(levels, dtype=np.float32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def cq_version():
    return int(_lib.cq_version())


def cq_blob_bytes(bits, rows, cols, group=CQ_GROUP):
    out = _u64(0)
    _check(_lib.cq_blob_bytes(bits, group, rows, cols, ctypes.byref(out)))
    return int(out.value)


@dataclass
class CQMatrix:
    """A CQ matrix: ``blob`` is a uint8 device tensor laid out as in cq.h;
    ``levels`` the host fp32 codebook (None for the ternary marker 5)."""
    bits: int
    rows: int
    cols: int
    blob: torch.Tensor
    levels: Optional[np.ndarray] = None
    group: int = CQ_GROUP

    def _key(self):
        b = self.blob
        lv = None if self.levels is None else np.asarray(self.levels, dtype=np.float32).tobytes()
        return (self.bits, self.group, self.rows, self.cols, b.data_ptr(), b.numel(), b.dtype, b.is_cuda,
                b.is_contiguous(), lv)

    def _struct(self):
        """The C descriptor (and the levels array it points to), rebuilt only
        when a field, the blob tensor or the level values change."""
        key = self._key()
        cached = self.__dict__.get("_c_struct")
        if cached is not None and cached[0] == key:
            return cached[1], cached[2]
        arr, ptr = _levels_array(self.levels)
        if self.blob.dtype != torch.uint8:
            raise TypeError("blob must be uint8")
        m = _Matrix(self.bits, self.group, self.rows, self.cols, _dev(self.blob, "blob"),
                    self.blob.numel(), ptr)
        self.__dict__["_c_struct"] = (key, m, arr)  # arr stays alive with the descriptor
        self.__dict__["_ws_bytes"] = {}
        return m, arr


def cq_workspace_bytes(op, W, batch):
    m, keep = W._struct()
    memo = W.__dict__["_ws_bytes"]  # reset whenever the descriptor is rebuilt
    if (op, batch) not in memo:
        out = _u64(0)
        _check(_lib.cq_workspace_bytes(op, ctypes.byref(m), batch, ctypes.byref(out)))
        memo[(op, batch)] = int(out.value)
    return memo[(op, batch)]


def _padded(cols):
    return -(-cols // CQ_GROUP) * CQ_GROUP


def cq_rotate_acts(x, out_dtype=torch.float32, out=None):
    """xr = per-128-group H.x of a [batch, cols] activation; returns [batch, cols_pad]."""
    if x.dim() != 2:
        raise ValueError("x must be [batch, cols]")
    if x.dtype not in _DTYPES:
        raise TypeError("x must be float32, float16 or bfloat16")
    b, cols = x.shape
    if out is None:
        out = torch.empty((b, _padded(cols)), dtype=out_dtype, device=x.device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    if tuple(out.shape) != (b, _padded(cols)):
        raise ValueError("out must be [batch, cols_pad]")
    _check(_lib.cq_rotate_acts(_dev(x, "x"), _DTYPES[x.dtype], b, cols, _dev(out, "out"),
                               _DTYPES[out.dtype], _stream()))
    return out


_WORKSPACES = {}


def workspace_for(nbytes, device):
    """A device workspace of at least ``nbytes`` bytes, cached per (device,
    current stream).  libcq needs no particular contents in it, and calls on
    one stream never overlap, so the cached one is reused as is."""
    if nbytes == 0:
        return None
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def cq_matvec(W, xr, out=None, workspace=None):
    """y[b, r] = sum_g norm * <c[q], xr_g>; xr float32 [batch, cols_pad]; returns float32 [batch, rows].

    ``workspace``: a uint8 device tensor of at least cq_workspace_bytes()
    bytes (any contents), or None to use a cached one for the current stream."""
    if xr.dtype != torch.float32 or xr.dim() != 2 or xr.shape[1] != _padded(W.cols):
        raise ValueError("xr must be float32 [batch, cols_pad]")
    b = xr.shape[0]
    if out is None:
        out = torch.empty((b, W.rows), dtype=torch.float32, device=xr.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.rows):
        raise ValueError("out must be float32 [batch, rows]")
    m, keep = W._struct()
    if workspace is None and b > 0 and W.rows > 0:
        need = _u64(0)
        _check(_lib.cq_workspace_bytes(OP_MATVEC, ctypes.byref(m), b, ctypes.byref(need)))
        workspace = workspace_for(int(need.value), xr.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.cq_matvec(ctypes.byref(m), _dev(xr, "xr"), b, _dev(out, "out"), ws, wsb, _stream()))
    return out


def cq_rotate_matvec(W, x, out=None, workspace=None):
    """cq_matvec(W, cq_rotate_acts(x)) in one call; x float32 [batch, cols]
    (not rotated); returns float32 [batch, rows].  ``workspace``: at least
    cq_workspace_bytes(OP_ROTATE_MATVEC) bytes, or None for a cached one."""
    if x.dtype != torch.float32 or x.dim() != 2 or x.shape[1] != W.cols:
        raise ValueError("x must be float32 [batch, cols]")
    x = x.contiguous()
    b = x.shape[0]
    if out is None:
        out = torch.empty((b, W.rows), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.rows):
        raise ValueError("out must be float32 [batch, rows]")
    m, keep = W._struct()
    if workspace is None and b > 0 and W.rows > 0:
        workspace = workspace_for(cq_workspace_bytes(OP_ROTATE_MATVEC, W, b), x.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.cq_rotate_matvec(ctypes.byref(m), _dev(x, "x"), b, _dev(out, "out"), ws, wsb, _stream()))
    return out


def cq_rotate_matvec_noalloc(W, x, out):
    """cq_rotate_matvec with the library's static device scratch instead of
    a workspace: x float32 [batch, cols] (not rotated), out float32 [batch,
    rows] (the caller provides it; the call allocates nothing)."""
    if x.dtype != torch.float32 or x.dim() != 2 or x.shape[1] != W.cols or not x.is_contiguous():
        raise ValueError("x must be contiguous float32 [batch, cols]")
    b = x.shape[0]
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.rows) or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [batch, rows]")
    m, keep = W._struct()
    _check(_lib.cq_rotate_matvec_noalloc(ctypes.byref(m), _dev(x, "x"), b, _dev(out, "out"), _stream()))
    return out


def _structs(Ws):
    arr = (_Matrix * max(len(Ws), 1))()
    keep = []
    for i, W in enumerate(Ws):
        m, k = W._struct()
        arr[i] = m
        keep.append(k)
    return arr, keep  # keep the levels arrays alive for the call


def cq_rotate_multi_workspace_bytes(Ws, batch):
    arr, keep = _structs(Ws)
    out = _u64(0)
    _check(_lib.cq_rotate_multi_workspace_bytes(arr, len(Ws), batch, ctypes.byref(out)))
    return int(out.value)


def cq_rotate_multi_matvec(Ws, x, outs=None, workspace=None):
    """[cq_rotate_matvec(W, x) for W in Ws] with the rotation of x shared:
    x float32 [batch, cols] (not rotated), every W with that cols; returns
    the list of float32 [batch, W.rows] results.  ``workspace``: at least
    cq_rotate_multi_workspace_bytes(Ws, batch) bytes, or None for a cached one."""
    Ws = list(Ws)
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be float32 [batch, cols]")
    if any(W.cols != x.shape[1] for W in Ws):
        raise ValueError("every matrix must have x's cols")
    x = x.contiguous()
    b = x.shape[0]
    if outs is None:
        outs = [torch.empty((b, W.rows), dtype=torch.float32, device=x.device) for W in Ws]
    outs = list(outs)
    if len(outs) != len(Ws):
        raise ValueError("one output per matrix")
    for W, o in zip(Ws, outs):
        if o.dtype != torch.float32 or tuple(o.shape) != (b, W.rows):
            raise ValueError("each out must be float32 [batch, rows]")
    arr, keep = _structs(Ws)
    if workspace is None and b > 0 and Ws:
        workspace = workspace_for(cq_rotate_multi_workspace_bytes(Ws, b), x.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ys = (_vp * max(len(outs), 1))(*[_dev(o, "out").value for o in outs])
    _check(_lib.cq_rotate_multi_matvec(arr, len(Ws), _dev(x, "x"), b, ys, ws, wsb, _stream()))
    return outs


def cq_quantize_acts_int8(x, xq=None, sx=None):
    """The rotated activation quantised per 128-group to int8: x float32
    [batch, cols] (not rotated); returns (xq int8 [batch, cols_pad], sx
    float32 [batch, cols_pad / 128])."""
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be float32 [batch, cols]")
    x = x.contiguous()
    b, cols = x.shape
    kpad = _padded(cols)
    if xq is None:
        xq = torch.empty((b, kpad), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty((b, kpad // CQ_GROUP), dtype=torch.float32, device=x.device)
    if xq.dtype != torch.int8 or tuple(xq.shape) != (b, kpad):
        raise ValueError("xq must be int8 [batch, cols_pad]")
    if sx.dtype != torch.float32 or tuple(sx.shape) != (b, kpad // CQ_GROUP):
        raise ValueError("sx must be float32 [batch, cols_pad / 128]")
    _check(_lib.cq_quantize_acts_int8(_dev(x, "x"), b, cols, _dev(xq, "xq"), _dev(sx, "sx"), _stream()))
    return xq, sx


def cq_matvec_w2a8_quantized(W, xq, sx, out=None):
    """The CQ-W2A8 product from quantised activations (cq_quantize_acts_int8's
    xq int8 [batch, cols_pad] and sx float32 [batch, cols_pad / 128]);
    returns float32 [batch, rows]."""
    kpad = _padded(W.cols)
    if xq.dtype != torch.int8 or xq.dim() != 2 or xq.shape[1] != kpad:
        raise ValueError("xq must be int8 [batch, cols_pad]")
    b = xq.shape[0]
    if sx.dtype != torch.float32 or tuple(sx.shape) != (b, kpad // CQ_GROUP):
        raise ValueError("sx must be float32 [batch, cols_pad / 128]")
    if out is None:
        out = torch.empty((b, W.rows), dtype=torch.float32, device=xq.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.rows):
        raise ValueError("out must be float32 [batch, rows]")
    m, keep = W._struct()
    _check(_lib.cq_matvec_w2a8_quantized(ctypes.byref(m), _dev(xq, "xq"), _dev(sx, "sx"), b, _dev(out, "out"),
                                         _stream()))
    return out


def cq_matvec_w2a8(W, x, out=None, workspace=None):
    """The CQ-W2A8 product (int8 activations and code book, integer dots, one
    float multiply per group) of x float32 [batch, cols] (not rotated);
    returns float32 [batch, rows].  ``workspace``: at least
    cq_workspace_bytes(OP_W2A8) bytes, or None for a cached one."""
    if x.dtype != torch.float32 or x.dim() != 2 or x.shape[1] != W.cols:
        raise ValueError("x must be float32 [batch, cols]")
    x = x.contiguous()
    b = x.shape[0]
    if out is None:
        out = torch.empty((b, W.rows), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.rows):
        raise ValueError("out must be float32 [batch, rows]")
    m, keep = W._struct()
    if workspace is None and b > 0 and W.rows > 0:
        workspace = workspace_for(cq_workspace_bytes(OP_W2A8, W, b), x.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.cq_matvec_w2a8(ctypes.byref(m), _dev(x, "x"), b, _dev(out, "out"), ws, wsb, _stream()))
    return out


def cq_gather_rows(W, ids, out_dtype=torch.float32, out=None):
    """Dense rows ``ids`` (int64 device tensor [n]) of the reconstruction;
    returns [n, cols] of out_dtype (float32, float16 or bfloat16).  Ids
    outside the matrix give rows of NaN."""
    if ids.dtype != torch.int64 or ids.dim() != 1:
        raise ValueError("ids must be an int64 vector")
    if out_dtype not in _DTYPES:
        raise TypeError("out_dtype must be float32, float16 or bfloat16")
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, W.cols), dtype=out_dtype, device=ids.device)
    if out.dtype not in _DTYPES or tuple(out.shape) != (n, W.cols):
        raise ValueError("out must be [n, cols] of float32, float16 or bfloat16")
    m, keep = W._struct()
    _check(_lib.cq_gather_rows(ctypes.byref(m), _dev(ids.contiguous(), "ids"), n, _dev(out, "out"),
                               _DTYPES[out.dtype], _stream()))
    return out


def cq_gemm(W, xr, out=None, workspace=None):
    """C[m, r] = sum_k xr[m, k] * bf16(c[q] * norm); xr bfloat16 [m, cols_pad]; returns float32 [m, rows]."""
    if xr.dtype != torch.bfloat16 or xr.dim() != 2 or xr.shape[1] != _padded(W.cols):
        raise ValueError("xr must be bfloat16 [m, cols_pad]")
    mrows = xr.shape[0]
    if out is None:
        out = torch.empty((mrows, W.rows), dtype=torch.float32, device=xr.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (mrows, W.rows):
        raise ValueError("out must be float32 [m, rows]")
    m, keep = W._struct()
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.cq_gemm(ctypes.byref(m), _dev(xr, "xr"), mrows, _dev(out, "out"), ws, wsb, _stream()))
    return out


def cq_quantize(w, bits, levels=None, group=CQ_GROUP, out=None):
    """Encode a float32 [rows, cols] device matrix; returns a CQMatrix whose blob is ``out``
    (allocated when None)."""
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be float32 [rows, cols]")
    rows, cols = w.shape
    nbytes = cq_blob_bytes(bits, rows, cols, group)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if out.dtype != torch.uint8 or out.numel() != nbytes:
        raise ValueError("out must be a uint8 tensor of cq_blob_bytes() bytes")
    arr, ptr = _levels_array(levels)
    _check(_lib.cq_quantize(_dev(w, "w"), rows, cols, bits, group, ptr, _dev(out, "out"), nbytes, _stream()))
    return CQMatrix(bits, rows, cols, out, arr, group)


def cq_quantize_rows(W, w, row0):
    """Encode w (float32 device [n, W.cols]) into rows row0 .. row0+n-1 of the
    existing matrix W (its blob is overwritten there): the append of new
    tokens to a CQ-quantised KV cache."""
    if w.dtype != torch.float32 or w.dim() != 2 or w.shape[1] != W.cols:
        raise ValueError("w must be float32 [n, cols]")
    m, keep = W._struct()
    _check(_lib.cq_quantize_rows(_dev(w.contiguous(), "w"), w.shape[0], ctypes.byref(m), row0, _stream()))
    return W


def cq_kv_scores_workspace_bytes(K, n_q_heads, n_kv_heads, head_dim):
    m, keep = K._struct()
    out = _u64(0)
    _check(_lib.cq_kv_scores_workspace_bytes(ctypes.byref(m), n_q_heads, n_kv_heads, head_dim, ctypes.byref(out)))
    return int(out.value)


def cq_kv_scores(K, q, n_kv_heads, out=None, workspace=None):
    """Scores of query heads q (float32 [n_q_heads, head_dim]) against the CQ
    key cache K [tokens, n_kv_heads * head_dim]; returns float32 [n_q_heads,
    tokens] (consecutive query heads share a KV head)."""
    if q.dtype != torch.float32 or q.dim() != 2:
        raise ValueError("q must be float32 [n_q_heads, head_dim]")
    nq, hd = q.shape
    if out is None:
        out = torch.empty((nq, K.rows), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (nq, K.rows):
        raise ValueError("out must be float32 [n_q_heads, tokens]")
    if workspace is None:
        workspace = workspace_for(cq_kv_scores_workspace_bytes(K, nq, n_kv_heads, hd) + 256, q.device)
    ws, wsb = ctypes.c_void_p(0), 0
    if workspace is not None:
        base = workspace.data_ptr()
        pad = (-base) % 256  # the call wants a 256-byte aligned workspace
        ws, wsb = ctypes.c_void_p(base + pad), workspace.numel() * workspace.element_size() - pad
    m, keep = K._struct()
    _check(_lib.cq_kv_scores(ctypes.byref(m), _dev(q.contiguous(), "q"), nq, n_kv_heads, hd, _dev(out, "out"),
                             ws, wsb, _stream()))
    return out


def cq_matvec_t(W, p, out=None, workspace=None):
    """out[b, k] = sum_r p[b, r] * w_hat[r, k]: p float32 [batch, rows];
    returns float32 [batch, cols] (the value side of attention over a CQ
    value cache)."""
    if p.dtype != torch.float32 or p.dim() != 2 or p.shape[1] != W.rows:
        raise ValueError("p must be float32 [batch, rows]")
    b = p.shape[0]
    if out is None:
        out = torch.empty((b, W.cols), dtype=torch.float32, device=p.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (b, W.cols):
        raise ValueError("out must be float32 [batch, cols]")
    if workspace is None and b > 0:
        workspace = workspace_for(cq_workspace_bytes(OP_MATVEC_T, W, b), p.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    m, keep = W._struct()
    _check(_lib.cq_matvec_t(ctypes.byref(m), _dev(p.contiguous(), "p"), b, _dev(out, "out"), ws, wsb, _stream()))
    return out


def cq_kv_append(K, V, k, v, row0):
    """Append n new tokens' keys k and values v (float32 [n, cols]) to the CQ
    caches K and V at rows row0 .. row0 + n - 1 (one launch when they share
    the code book).  Returns (K, V)."""
    for name, t, M in (("k", k, K), ("v", v, V)):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != M.cols:
            raise ValueError(f"{name} must be float32 [n, cols]")
    if k.shape[0] != v.shape[0]:
        raise ValueError("k and v must hold the same number of rows")
    mk, keep_k = K._struct()
    mv, keep_v = V._struct()
    _check(_lib.cq_kv_append(ctypes.byref(mk), ctypes.byref(mv), _dev(k.contiguous(), "k"), _dev(v.contiguous(), "v"),
                             k.shape[0], row0, _stream()))
    return K, V


def cq_kv_attention(K, V, q, n_kv_heads, tokens=None, scale=None, out=None):
    """One decode attention step: query heads q (float32 [n_q_heads,
    head_dim]) against the first ``tokens`` rows (default: all) of the CQ key
    and value caches K, V [rows, n_kv_heads * head_dim]; softmax of ``scale``
    (default 1/sqrt(head_dim)) times the scores, then the weighted value rows.
    Returns float32 [n_q_heads, head_dim]."""
    if q.dtype != torch.float32 or q.dim() != 2:
        raise ValueError("q must be float32 [n_q_heads, head_dim]")
    nq, hd = q.shape
    tokens = K.rows if tokens is None else int(tokens)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    if out is None:
        out = torch.empty((nq, hd), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (nq, hd):
        raise ValueError("out must be float32 [n_q_heads, head_dim]")
    mk, keep_k = K._struct()
    mv, keep_v = V._struct()
    _check(_lib.cq_kv_attention(ctypes.byref(mk), ctypes.byref(mv), tokens, _dev(q.contiguous(), "q"), nq,
                                n_kv_heads, hd, scale, _dev(out, "out"), _stream()))
    return out


def cq_read_probe(buf, sink):
    """Read every byte of ``buf`` (a device tensor) once with plain wide loads
    (the streaming-read ceiling); ``sink`` is a uint32/int32 device tensor of
    a multiple of 256 words (one workgroup per 256)."""
    _check(_lib.cq_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"),
                              sink.numel() * sink.element_size() // 4, _stream()))
