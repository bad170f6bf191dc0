"""Thin Python binding of libsaga.so (ctypes): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels. PyTorch provides
device memory (tensor storage) and the stream (torch's current stream). If the
library is not built, every call raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import LIB_PATH

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)
F32, BF16 = 0, 1
EXPORTS = ("saga_status_str", "saga_workspace_bytes", "saga_workspace_init", "saga_decode_attn",
           "saga_refresh_threshold", "saga_dense_gqa_attn", "saga_qk_select", "saga_sparse_gather",
           "saga_select_gather", "saga_split_combine", "saga_decode_attn_paged", "saga_dense_gqa_attn_paged",
           "saga_linear", "saga_qkv_append", "saga_layer_workspace_bytes", "saga_decode_layer",
           "saga_merge_workspace_bytes", "saga_merge_losses", "saga_min_weight_pairing", "saga_merge_keys",
           "saga_decode_attn_noalloc", "saga_gather_form")
NOALLOC_SCRATCH_BYTES = 64 << 20  # SAGA_NOALLOC_SCRATCH_BYTES of include/saga.h
ATTN_ATOPN, ATTN_DENSE = 0, 1
FLAG_REFRESHED, FLAG_FORCED = 1, 2


class SagaShape(ctypes.Structure):
    """Mirror of `saga_shape` in include/saga.h."""
    _fields_ = [("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_k", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d", ctypes.c_int32), ("d_v", ctypes.c_int32), ("l_max", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class SagaPages(ctypes.Structure):
    """Mirror of `saga_pages` in include/saga.h."""
    _fields_ = [("table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class SagaLayer(ctypes.Structure):
    """Mirror of `saga_layer` in include/saga.h."""
    _fields_ = [("attn", SagaShape), ("d_model", ctypes.c_int32)]


class SagaMergeShape(ctypes.Structure):
    """Mirror of `saga_merge_shape` in include/saga.h."""
    _fields_ = [("tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_k", ctypes.c_int32), ("d", ctypes.c_int32)]


class SagaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)}")
        self.status = status


_LIB = None
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "saga_status_str": (ctypes.c_char_p, [_I32]),
    "saga_workspace_bytes": (_SZ, [_P, _I32, _I32]),
    "saga_gather_form": (_I32, [_P, _I32, _I32]),
    "saga_workspace_init": (_I32, [_P, _SZ, _P]),
    "saga_decode_attn": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_decode_attn_noalloc": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _P, _P]),
    "saga_refresh_threshold": (_I32, [_P, _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "saga_dense_gqa_attn": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_qk_select": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_sparse_gather": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_select_gather": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "saga_split_combine": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_decode_attn_paged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _P, _P,
                                      _SZ, _P]),
    "saga_dense_gqa_attn_paged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "saga_linear": (_I32, [_I32, _I32, _I32, _P, _P, _P, _I32, _P]),
    "saga_qkv_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "saga_layer_workspace_bytes": (_SZ, [_P, _I32, _I32]),
    "saga_decode_layer": (_I32, [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P,
                                 _SZ, _P]),
    "saga_merge_workspace_bytes": (_SZ, [_P]),
    "saga_merge_losses": (_I32, [_P, _P, _P, _P, _P, _P, _SZ, _P]),
    "saga_min_weight_pairing": (_I32, [_I32, _P, _P, _P]),
    "saga_merge_keys": (_I32, [_P, _P, _P, _P, _P, _SZ, _P]),
}


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsaga.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m sparse_decode_attention_saga_amd.build`")
        cdll = ctypes.CDLL(p)
        for name, (res, args) in _SIGS.items():
            fn = getattr(cdll, name)
            fn.restype, fn.argtypes = res, args
        _LIB = cdll
    return _LIB


def status_str(status: int) -> str:
    return lib().saga_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise SagaError(status, where)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {dt}: use float32 or bfloat16")


def make_shape(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None,
               out_dtype: Optional[torch.dtype] = None, scale: float = 0.0, d_v: int = 0) -> SagaShape:
    """Shape of q [B, h_q, d], k [B, h_k, l_max, d] and v [B, h_v, l_max, d_v]. Without
    v, `d_v` gives the value head dimension (0: d)."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, h_q, d] and k [B, h_k, l_max, d]")
    B, h_q, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k does not match q")
    h_v = k.shape[1]
    if v is not None:
        if v.dim() != 4 or v.shape[0] != B or v.shape[2] != k.shape[2]:
            raise ValueError("v must be [B, h_v, l_max, d_v] matching k")
        if v.dtype != q.dtype:
            raise ValueError("q, k and v must share one dtype")
        h_v = v.shape[1]
        d_v = v.shape[3]
    if k.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    return SagaShape(B, h_q, k.shape[1], h_v, d, 0 if d_v == d else int(d_v), k.shape[2], dtype_code(q.dtype),
                     dtype_code(out_dtype or q.dtype), float(scale))


def value_dim(shape: SagaShape) -> int:
    return shape.d_v if shape.d_v > 0 else shape.d


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def workspace_bytes(shape: SagaShape, N: int, max_l_kv: int) -> int:
    n = lib().saga_workspace_bytes(ctypes.byref(shape), int(N), int(max_l_kv))
    if n == 0:
        raise ValueError("invalid shape for the workspace")
    return int(n)


def gather_form(shape: SagaShape, N: int, max_l_kv: int) -> str:
    """"late" or "early": where the decode step gathers the kept value rows (saga_gather_form)."""
    f = lib().saga_gather_form(ctypes.byref(shape), int(N), int(max_l_kv))
    if f < 0:
        raise ValueError("invalid shape, N or max_l_kv")
    return "late" if f == 1 else "early"


class Workspace:
    """Device workspace for one shape: zero-filled once by the library's fill kernel."""

    def __init__(self, shape: SagaShape, N: int, max_l_kv: int, device, stream=None):
        self.nbytes = workspace_bytes(shape, N, max_l_kv)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _check(lib().saga_workspace_init(_ptr(self.buf), self.nbytes, _stream(self.buf.device, stream)),
               "saga_workspace_init")

    @classmethod
    def for_inputs(cls, q, k, v=None, N: int = 1, max_l_kv: Optional[int] = None):
        shape = make_shape(q, k, v)
        return cls(shape, N, k.shape[2] if max_l_kv is None else max_l_kv, q.device)


def _prep(q, k, v, l_kv, tau, out, out_dtype, max_l_kv, scale, d_v=0, need_out=True):
    """Checks the tensors of a call and returns (shape, max_l_kv, out); without
    `need_out` the call writes no output and `out` is None."""
    for name, t in (("q", q), ("k", k)):
        _dev(t, name)
    if v is not None:
        _dev(v, "v")
    _dev(l_kv, "l_kv", torch.int32)
    if out_dtype is None and out is not None:
        out_dtype = out.dtype
    shape = make_shape(q, k, v, out_dtype, scale, d_v)
    if l_kv.numel() != shape.batch:
        raise ValueError("l_kv must have one entry per sequence")
    if tau is not None:
        _dev(tau, "tau", torch.float32)
        if tau.numel() != shape.batch * shape.h_q:
            raise ValueError("tau must be [B, h_q]")
    if l_kv.device != q.device or (tau is not None and tau.device != q.device):
        raise ValueError("every tensor of a call must be on one device")
    if max_l_kv is None:
        max_l_kv = shape.l_max
    out_shape = (shape.batch, shape.h_q, value_dim(shape))
    if not need_out:
        return shape, int(max_l_kv), None
    if out is None:
        out = torch.empty(out_shape, dtype=out_dtype or q.dtype, device=q.device)
    else:
        _dev(out, "out")
        if tuple(out.shape) != out_shape or dtype_code(out.dtype) != shape.out_dtype:
            raise ValueError("out must be [B, h_q, d_v] in the output dtype")
    return shape, int(max_l_kv), out


def _row_outputs(B: int, h_q: int, sel_count, sel_idx, flags) -> int:
    """Checks the optional per-(sequence, query head) outputs: sel_count and flags
    [B, h_q] int32, sel_idx [B, h_q, cap] int32. Returns cap (0 without sel_idx).
    The kernels write B*h_q counts and flags and cap indices per row, so a smaller
    tensor is refused here rather than written past its end."""
    for name, t in (("sel_count", sel_count), ("flags", flags)):
        if t is not None:
            _dev(t, name, torch.int32)
            if t.numel() != B * h_q:
                raise ValueError(f"{name} must be [B, h_q] = [{B}, {h_q}]")
    if sel_idx is None:
        return 0
    _dev(sel_idx, "sel_idx", torch.int32)
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (B, h_q) or sel_idx.shape[2] < 1:
        raise ValueError(f"sel_idx must be [B, h_q, cap] = [{B}, {h_q}, cap >= 1]")
    return int(sel_idx.shape[2])


def _ws(ws: Optional[Workspace], shape, N, max_l_kv, device):
    if ws is None:
        ws = Workspace(shape, N, max_l_kv, device)
    return ws


def decode_attn(q, k, v, l_kv, tau, *, N: int, refresh_period: int, step: int,
                max_l_kv: Optional[int] = None, out=None, out_dtype=None, sel_count=None,
                sel_idx=None, flags=None, workspace: Optional[Workspace] = None,
                scale: float = 0.0, stream=None):
    """saga_decode_attn: one SAGA + Atop-N decode step. `tau` [B, h_q] float32 is
    read and updated in place. Returns `out`."""
    shape, max_l_kv, out = _prep(q, k, v, l_kv, tau, out, out_dtype, max_l_kv, scale)
    cap = _row_outputs(shape.batch, shape.h_q, sel_count, sel_idx, flags)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv, int(N),
                                int(refresh_period), int(step), _ptr(tau), _ptr(out), _ptr(sel_count),
                                _ptr(sel_idx), cap, _ptr(flags), _ptr(ws.buf), ws.nbytes,
                                _stream(q.device, stream))
    _check(st, "saga_decode_attn")
    return out


def decode_attn_noalloc(q, k, v, l_kv, tau, *, N: int, refresh_period: int, step: int,
                        max_l_kv: Optional[int] = None, out=None, sel_count=None, sel_idx=None, flags=None,
                        scale: float = 0.0, stream=None):
    """saga_decode_attn_noalloc: decode_attn with the library's own per-GPU scratch
    instead of a workspace (nothing is allocated by the library). `out` must be given,
    so that the call allocates nothing here either. Returns `out`."""
    if out is None:
        raise ValueError("decode_attn_noalloc needs a preallocated out [B, h_q, d_v]")
    shape, max_l_kv, out = _prep(q, k, v, l_kv, tau, out, None, max_l_kv, scale)
    cap = _row_outputs(shape.batch, shape.h_q, sel_count, sel_idx, flags)
    st = lib().saga_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv,
                                        int(N), int(refresh_period), int(step), _ptr(tau), _ptr(out),
                                        _ptr(sel_count), _ptr(sel_idx), cap, _ptr(flags), _stream(q.device, stream))
    _check(st, "saga_decode_attn_noalloc")
    return out


def refresh_threshold(q, k, l_kv, tau, *, N: int, max_l_kv: Optional[int] = None,
                      workspace: Optional[Workspace] = None, scale: float = 0.0, d_v: int = 0, stream=None):
    """saga_refresh_threshold: writes the exact threshold into `tau` [B, h_q]. `d_v`:
    the value head dimension of the caches (0: that of q and k)."""
    shape, max_l_kv, _ = _prep(q, k, None, l_kv, tau, None, None, max_l_kv, scale, d_v, need_out=False)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_refresh_threshold(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(l_kv), max_l_kv, int(N),
                                      _ptr(tau), _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_refresh_threshold")
    return tau


def qk_select(q, k, l_kv, tau, *, max_l_kv: Optional[int] = None, workspace: Optional[Workspace] = None,
              scale: float = 0.0, d_v: int = 0, stream=None):
    """saga_qk_select: the scoring and threshold-comparison stage (into the workspace).
    `d_v`: the value head dimension of the caches (0: that of q and k)."""
    shape, max_l_kv, _ = _prep(q, k, None, l_kv, tau, None, None, max_l_kv, scale, d_v, need_out=False)
    ws = _ws(workspace, shape, 1, max_l_kv, q.device)
    st = lib().saga_qk_select(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(l_kv), max_l_kv, _ptr(tau),
                              _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_qk_select")


def sparse_gather(q, k, v, l_kv, tau, *, N: int, max_l_kv: Optional[int] = None, out=None, out_dtype=None,
                  sel_count=None, sel_idx=None, flags=None, workspace: Optional[Workspace] = None,
                  scale: float = 0.0, stream=None):
    """saga_sparse_gather: softmax and value gather over what saga_qk_select kept."""
    shape, max_l_kv, out = _prep(q, k, v, l_kv, tau, out, out_dtype, max_l_kv, scale)
    cap = _row_outputs(shape.batch, shape.h_q, sel_count, sel_idx, flags)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_sparse_gather(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv, int(N),
                                  _ptr(tau), _ptr(out), _ptr(sel_count), _ptr(sel_idx), cap, _ptr(flags),
                                  _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_sparse_gather")
    return out


def select_gather(q, k, v, l_kv, tau, *, N: int, max_l_kv: Optional[int] = None,
                  workspace: Optional[Workspace] = None, scale: float = 0.0, stream=None):
    """saga_select_gather: scoring, threshold comparison and, per chunk, either the parts
    of the softmax-weighted value sum (early gather) or the kept (index, logit) pairs
    (late gather), into the workspace; N chooses the form as in decode_attn."""
    shape, max_l_kv, _ = _prep(q, k, v, l_kv, tau, None, None, max_l_kv, scale, need_out=False)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_select_gather(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv, int(N),
                                  _ptr(tau), _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_select_gather")


def split_combine(q, k, v, l_kv, tau, *, N: int, max_l_kv: Optional[int] = None, out=None, out_dtype=None,
                  sel_count=None, sel_idx=None, flags=None, workspace: Optional[Workspace] = None,
                  scale: float = 0.0, stream=None):
    """saga_split_combine: eq. (7) into `out` from what saga_select_gather left (same N)."""
    shape, max_l_kv, out = _prep(q, k, v, l_kv, tau, out, out_dtype, max_l_kv, scale)
    cap = _row_outputs(shape.batch, shape.h_q, sel_count, sel_idx, flags)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_split_combine(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv, int(N),
                                  _ptr(tau), _ptr(out), _ptr(sel_count), _ptr(sel_idx), cap, _ptr(flags),
                                  _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_split_combine")
    return out


def dense_gqa_attn(q, k, v, l_kv, *, max_l_kv: Optional[int] = None, out=None, out_dtype=None,
                   workspace: Optional[Workspace] = None, scale: float = 0.0, stream=None):
    """saga_dense_gqa_attn: dense grouped-query attention over every cached key (h_k == h_v)."""
    shape, max_l_kv, out = _prep(q, k, v, l_kv, None, out, out_dtype, max_l_kv, scale)
    ws = _ws(workspace, shape, 1, max_l_kv, q.device)
    st = lib().saga_dense_gqa_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(l_kv), max_l_kv,
                                   _ptr(out), _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_dense_gqa_attn")
    return out


def _prep_paged(q, k_pages, v_pages, table, l_kv, tau, out, out_dtype, max_l_kv, scale):
    """Shape and page descriptor of a paged call: k_pages [num_pages, h_k, P, d],
    v_pages [num_pages, h_v, P, d_v], table [B, max_pages] int32."""
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _dev(t, name)
    _dev(table, "table", torch.int32)
    _dev(l_kv, "l_kv", torch.int32)
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.dim() != 4 or table.dim() != 2:
        raise ValueError("q [B, h_q, d], k_pages [num_pages, h_k, page_tokens, d], "
                         "v_pages [num_pages, h_v, page_tokens, d_v], table [B, max_pages]")
    B, h_q, d = q.shape
    num_pages, h_k, P, dk = k_pages.shape
    d_v = v_pages.shape[3]
    if v_pages.shape[0] != num_pages or v_pages.shape[2] != P or dk != d:
        raise ValueError("k_pages and v_pages must share num_pages and page_tokens, and k_pages d with q")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise ValueError("q, k_pages and v_pages must share one dtype")
    if table.shape[0] != B or l_kv.numel() != B:
        raise ValueError("table and l_kv need one row per sequence")
    capacity = table.shape[1] * P
    if max_l_kv is None:
        max_l_kv = capacity
    if out_dtype is None and out is not None:
        out_dtype = out.dtype
    shape = SagaShape(B, h_q, h_k, v_pages.shape[1], d, 0 if d_v == d else d_v, max(int(max_l_kv), 1),
                      dtype_code(q.dtype), dtype_code(out_dtype or q.dtype), float(scale))
    pages = SagaPages(table.data_ptr(), table.shape[1], P, num_pages)
    if tau is not None:
        _dev(tau, "tau", torch.float32)
        if tau.numel() != B * h_q:
            raise ValueError("tau must be [B, h_q]")
    if out is None:
        out = torch.empty((B, h_q, d_v), dtype=out_dtype or q.dtype, device=q.device)
    else:
        _dev(out, "out")
        if tuple(out.shape) != (B, h_q, d_v) or dtype_code(out.dtype) != shape.out_dtype:
            raise ValueError("out must be [B, h_q, d_v] in the output dtype")
    return shape, pages, int(max_l_kv), out


def decode_attn_paged(q, k_pages, v_pages, table, l_kv, tau, *, N: int, refresh_period: int, step: int,
                      max_l_kv: Optional[int] = None, out=None, out_dtype=None, sel_count=None, sel_idx=None,
                      flags=None, workspace: Optional[Workspace] = None, scale: float = 0.0, stream=None):
    """saga_decode_attn_paged: decode_attn over paged caches (pages of page_tokens
    tokens found through `table`). Returns `out`."""
    shape, pages, max_l_kv, out = _prep_paged(q, k_pages, v_pages, table, l_kv, tau, out, out_dtype, max_l_kv,
                                              scale)
    cap = _row_outputs(shape.batch, shape.h_q, sel_count, sel_idx, flags)
    ws = _ws(workspace, shape, N, max_l_kv, q.device)
    st = lib().saga_decode_attn_paged(ctypes.byref(shape), ctypes.byref(pages), _ptr(q), _ptr(k_pages),
                                      _ptr(v_pages), _ptr(l_kv), max_l_kv, int(N), int(refresh_period), int(step),
                                      _ptr(tau), _ptr(out), _ptr(sel_count), _ptr(sel_idx), cap, _ptr(flags),
                                      _ptr(ws.buf), ws.nbytes, _stream(q.device, stream))
    _check(st, "saga_decode_attn_paged")
    return out


def dense_gqa_attn_paged(q, k_pages, v_pages, table, l_kv, *, max_l_kv: Optional[int] = None, out=None,
                         out_dtype=None, workspace: Optional[Workspace] = None, scale: float = 0.0, stream=None):
    """saga_dense_gqa_attn_paged: dense attention over paged caches."""
    shape, pages, max_l_kv, out = _prep_paged(q, k_pages, v_pages, table, l_kv, None, out, out_dtype, max_l_kv,
                                              scale)
    ws = _ws(workspace, shape, 1, max_l_kv, q.device)
    st = lib().saga_dense_gqa_attn_paged(ctypes.byref(shape), ctypes.byref(pages), _ptr(q), _ptr(k_pages),
                                         _ptr(v_pages), _ptr(l_kv), max_l_kv, _ptr(out), _ptr(ws.buf), ws.nbytes,
                                         _stream(q.device, stream))
    _check(st, "saga_dense_gqa_attn_paged")
    return out


# --- decode layer (eq. (1) projections, cache append, attention, W_O) -------------

def linear(x, w, *, out=None, out_dtype=None, stream=None):
    """saga_linear: y = x w^T for x [B, n_in] and w [n_out, n_in], both bfloat16."""
    _dev(x, "x", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [B, n_in] and w [n_out, n_in]")
    B, n_out = x.shape[0], w.shape[0]
    if out is None:
        out = torch.empty(B, n_out, dtype=out_dtype or torch.bfloat16, device=x.device)
    else:
        _dev(out, "out")
        if tuple(out.shape) != (B, n_out):
            raise ValueError("out must be [B, n_out]")
    st = lib().saga_linear(B, x.shape[1], n_out, _ptr(x), _ptr(w), _ptr(out), dtype_code(out.dtype),
                           _stream(x.device, stream))
    _check(st, "saga_linear")
    return out


def layer_desc(x, k_cache, v_cache, h_q: int, out_dtype=None, scale: float = 0.0) -> SagaLayer:
    """The layer descriptor for x [B, d_model] and caches [B, h_k, l_max, d], [B, h_v, l_max, d]."""
    if x.dim() != 2 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("x must be [B, d_model], caches [B, heads, l_max, d]")
    B, h_k, l_max, d = k_cache.shape
    if v_cache.shape[0] != B or v_cache.shape[2:] != k_cache.shape[2:] or x.shape[0] != B:
        raise ValueError("x, k_cache and v_cache disagree")
    for t in (x, k_cache, v_cache):
        if t.dtype != torch.bfloat16:
            raise ValueError("the layer computes in bfloat16")
    shape = SagaShape(B, h_q, h_k, v_cache.shape[1], d, 0, l_max, BF16, dtype_code(out_dtype or torch.bfloat16),
                      float(scale))
    return SagaLayer(shape, x.shape[1])


def qkv_append(x, w_qkv, k_cache, v_cache, l_kv, l_kv_next, *, h_q: int, q=None, stream=None):
    """saga_qkv_append: q (returned, [B, h_q, d] bf16) and the new cache rows."""
    for name, t in (("x", x), ("w_qkv", w_qkv), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, torch.bfloat16)
    _dev(l_kv, "l_kv", torch.int32)
    _dev(l_kv_next, "l_kv_next", torch.int32)
    L = layer_desc(x, k_cache, v_cache, h_q)
    if tuple(w_qkv.shape) != ((h_q + L.attn.h_k + L.attn.h_v) * L.attn.d, L.d_model):
        raise ValueError("w_qkv must be [(h_q + h_k + h_v) * d, d_model]")
    if l_kv.numel() != x.shape[0] or l_kv_next.numel() != x.shape[0]:
        raise ValueError("l_kv and l_kv_next need one entry per sequence")
    if q is None:
        q = torch.empty(x.shape[0], h_q, L.attn.d, dtype=torch.bfloat16, device=x.device)
    else:
        _dev(q, "q", torch.bfloat16)
        if tuple(q.shape) != (x.shape[0], h_q, L.attn.d):
            raise ValueError("q must be [B, h_q, d]")
    st = lib().saga_qkv_append(ctypes.byref(L), _ptr(x), _ptr(w_qkv), _ptr(k_cache), _ptr(v_cache), _ptr(l_kv),
                               _ptr(l_kv_next), _ptr(q), _stream(x.device, stream))
    _check(st, "saga_qkv_append")
    return q


class LayerWorkspace:
    """Device workspace of saga_decode_layer, zero-filled once."""

    def __init__(self, L: SagaLayer, N: int, max_l_kv: int, device, stream=None):
        n = lib().saga_layer_workspace_bytes(ctypes.byref(L), int(N), int(max_l_kv))
        if n == 0:
            raise ValueError("invalid layer shape for the workspace")
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _check(lib().saga_workspace_init(_ptr(self.buf), self.nbytes, _stream(self.buf.device, stream)),
               "saga_workspace_init")


def decode_layer(x, w_qkv, w_o, k_cache, v_cache, l_kv, l_kv_next, *, h_q: int, attention: int = ATTN_ATOPN,
                 N: int = 1, refresh_period: int = 1, step: int = 0, tau=None, max_l_kv: Optional[int] = None,
                 out=None, out_dtype=None, sel_count=None, flags=None, workspace: Optional[LayerWorkspace] = None,
                 scale: float = 0.0, stream=None):
    """saga_decode_layer: one decode layer for the new token x [B, d_model]; returns y [B, d_model]."""
    for name, t in (("x", x), ("w_qkv", w_qkv), ("w_o", w_o), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, torch.bfloat16)
    _dev(l_kv, "l_kv", torch.int32)
    _dev(l_kv_next, "l_kv_next", torch.int32)
    if out_dtype is None and out is not None:
        out_dtype = out.dtype
    L = layer_desc(x, k_cache, v_cache, h_q, out_dtype, scale)
    if tuple(w_qkv.shape) != ((h_q + L.attn.h_k + L.attn.h_v) * L.attn.d, L.d_model):
        raise ValueError("w_qkv must be [(h_q + h_k + h_v) * d, d_model]")
    if tuple(w_o.shape) != (L.d_model, h_q * L.attn.d):
        raise ValueError("w_o must be [d_model, h_q * d]")
    B = x.shape[0]
    if l_kv.numel() != B or l_kv_next.numel() != B:
        raise ValueError("l_kv and l_kv_next need one entry per sequence")
    if attention == ATTN_ATOPN and tau is None:
        raise ValueError("the Atop-N layer needs the threshold state tau [B, h_q]")
    if tau is not None:
        _dev(tau, "tau", torch.float32)
        if tau.numel() != B * h_q:
            raise ValueError("tau must be [B, h_q]")
    _row_outputs(B, h_q, sel_count, None, flags)
    if max_l_kv is None:
        max_l_kv = L.attn.l_max
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or torch.bfloat16, device=x.device)
    else:
        _dev(out, "out")
        if tuple(out.shape) != tuple(x.shape) or dtype_code(out.dtype) != L.attn.out_dtype:
            raise ValueError("out must be [B, d_model] in the output dtype")
    n = N if attention == ATTN_ATOPN else 1
    ws = workspace or LayerWorkspace(L, n, max_l_kv, x.device)
    st = lib().saga_decode_layer(ctypes.byref(L), int(attention), _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(l_kv), _ptr(l_kv_next), int(max_l_kv), int(N),
                                 int(refresh_period), int(step), _ptr(tau), _ptr(out), _ptr(sel_count),
                                 _ptr(flags), _ptr(ws.buf), ws.nbytes, _stream(x.device, stream))
    _check(st, "saga_decode_layer")
    return out


# --- GQA-to-SAGA key-head merge (closed-form initialisation) ------------------------

class MergeWorkspace:
    """Device workspace of the merge calls (no zero fill needed)."""

    def __init__(self, shape: SagaMergeShape, device):
        n = lib().saga_merge_workspace_bytes(ctypes.byref(shape))
        if n == 0:
            raise ValueError("invalid merge shape")
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)


def merge_shape(x, w_q, w_k, h_q: int, h_k: int) -> SagaMergeShape:
    """Shape of x [T, D], w_q [h_q d, D], w_k [h_k d, D] (bfloat16, transposed projections)."""
    if x.dim() != 2 or w_q.dim() != 2 or w_k.dim() != 2:
        raise ValueError("x [tokens, d_model], w_q [h_q*d, d_model], w_k [h_k*d, d_model]")
    T, D = x.shape
    if w_q.shape[1] != D or w_k.shape[1] != D or w_q.shape[0] % h_q or w_k.shape[0] % h_k:
        raise ValueError("w_q and w_k must be [heads*d, d_model] matching x")
    d = w_q.shape[0] // h_q
    if w_k.shape[0] != h_k * d:
        raise ValueError("w_q and w_k must share the head dimension")
    return SagaMergeShape(T, D, h_q, h_k, d)


def merge_losses(x, w_q, w_k, *, h_q: int, h_k: int, workspace: Optional[MergeWorkspace] = None, stream=None):
    """saga_merge_losses: eq. (13) at eq. (15) for every pair of teacher key heads.
    Returns (loss [h_k, h_k] float32 on the device, the workspace holding the pairs'
    merge coefficients)."""
    for name, t in (("x", x), ("w_q", w_q), ("w_k", w_k)):
        _dev(t, name, torch.bfloat16)
    shape = merge_shape(x, w_q, w_k, h_q, h_k)
    ws = workspace or MergeWorkspace(shape, x.device)
    loss = torch.empty(h_k, h_k, dtype=torch.float32, device=x.device)
    st = lib().saga_merge_losses(ctypes.byref(shape), _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(loss), _ptr(ws.buf),
                                 ws.nbytes, _stream(x.device, stream))
    _check(st, "saga_merge_losses")
    return loss, ws


def min_weight_pairing(weight):
    """saga_min_weight_pairing (host): weight [n, n] (CPU float32 tensor or array-like).
    Returns (partner list, total weight)."""
    w = torch.as_tensor(weight, dtype=torch.float32).contiguous()
    if w.is_cuda or w.dim() != 2 or w.shape[0] != w.shape[1]:
        raise ValueError("weight must be a square host matrix")
    n = w.shape[0]
    partner = (ctypes.c_int32 * n)()
    total = ctypes.c_double(0.0)
    st = lib().saga_min_weight_pairing(n, ctypes.c_void_p(w.data_ptr()), partner, ctypes.byref(total))
    _check(st, "saga_min_weight_pairing")
    return list(partner), float(total.value)


def merge_keys(x, w_q, w_k, partner, *, h_q: int, h_k: int, workspace: MergeWorkspace, out=None, stream=None):
    """saga_merge_keys: merged key projections [h_k/2 * d, D] float32 for the pairing
    `partner` (host list), using the coefficients saga_merge_losses left in `workspace`."""
    _dev(w_k, "w_k", torch.bfloat16)
    shape = merge_shape(x, w_q, w_k, h_q, h_k)
    if len(partner) != h_k:
        raise ValueError("one partner per teacher key head")
    part = (ctypes.c_int32 * h_k)(*[int(p) for p in partner])
    if out is None:
        out = torch.empty(h_k // 2 * shape.d, shape.d_model, dtype=torch.float32, device=w_k.device)
    else:
        _dev(out, "out", torch.float32)
        if tuple(out.shape) != (h_k // 2 * shape.d, shape.d_model):
            raise ValueError("out must be [h_k/2 * d, d_model]")
    st = lib().saga_merge_keys(ctypes.byref(shape), _ptr(w_k), part, _ptr(out), _ptr(workspace.buf),
                               workspace.nbytes, _stream(w_k.device, stream))
    _check(st, "saga_merge_keys")
    return out


def merge_key_heads(x, w_q, w_k, *, h_q: int, h_k: int):
    """The whole closed-form initialisation: pair losses on the device, the pairing on
    the host (the loss matrix is copied back), the merged projections on the device.
    Returns (pairs [(a, b), ...], total loss, merged w_k [h_k/2 * d, D] float32, loss)."""
    loss, ws = merge_losses(x, w_q, w_k, h_q=h_q, h_k=h_k)
    partner, total = min_weight_pairing(loss.cpu())
    out = merge_keys(x, w_q, w_k, partner, h_q=h_q, h_k=h_k, workspace=ws)
    pairs = sorted((a, b) for a, b in enumerate(partner) if a < b)
    return pairs, total, out, loss
