"""Exact-attention forward for MI355X (gfx950): Python binding of the C ABI.

The functions ``fa_fwd``, ``fa_fwd_splitkv``, ``fa_fwd_splitkv_noalloc``,
``fa_splitkv_num_splits``, ``fa_splitkv_workspace_bytes``, ``fa_fwd_splitkv_qk``,
``fa_splitkv_qk_num_splits``, ``fa_splitkv_qk_workspace_bytes``, ``fa_merge_partials``,
``fa_softmax_rows``, ``fa_softmax_workspace_bytes``, ``fa_softmax_x_reads``,
``fa_softmax_set_wait_limit``, ``fa_bwd``, ``fa_bwd_workspace_bytes``,
``fa_fwd_fp8``, ``fa_naive_fwd``, ``fa_naive_workspace_bytes``,
``fa_status_string``, ``fa_last_error`` and ``fa_version`` carry the names and
meaning of the entry points declared in ``include/fa_api.h``; they only
marshal torch tensors into pointers, sizes and the current HIP stream.  Every
step of the computation runs in the HIP kernels of ``libiofa.so``; there is
no CPU fallback, and a missing library raises instead of computing.

``forward``, ``forward_splitkv``, ``forward_qk``, ``forward_fp8``, ``backward``,
``softmax`` and ``naive_forward`` are conveniences that allocate the outputs (and workspaces)
with torch and call the entry points.
"""

import ctypes
import math
import os

import numpy as np
import torch

__all__ = [
    "FA_F32", "FA_F16", "FA_BF16", "FaError", "library_path", "load_library",
    "fa_fwd", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "FA_NOALLOC_SCRATCH_BYTES",
    "fa_splitkv_num_splits", "fa_splitkv_workspace_bytes", "fa_fwd_splitkv_qk",
    "fa_splitkv_qk_num_splits", "fa_splitkv_qk_workspace_bytes", "forward_qk",
    "fa_merge_partials", "fa_softmax_rows", "fa_softmax_workspace_bytes", "fa_softmax_x_reads",
    "fa_softmax_set_wait_limit", "softmax",
    "fa_bwd", "fa_bwd_workspace_bytes", "backward", "fa_fwd_fp8", "forward_fp8",
    "fa_naive_fwd", "fa_naive_workspace_bytes", "fa_status_string",
    "fa_last_error", "fa_version", "forward", "forward_splitkv", "naive_forward",
    "default_scale",
]

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libiofa.so")
_lib = None


class FaError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{fa_status_string(status)} (status {status}): {detail}")


def library_path():
    return _LIB_PATH


def load_library():
    """Load libiofa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built: run `python -m io_aware_softmax_04_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, fp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, fp, i64, i64, i64, i64, ctypes.c_float,
                           ctypes.c_int, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, fp, i64, i64, i64, i64, ctypes.c_float,
                               ctypes.c_float, ctypes.c_float, ctypes.c_float, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, fp, vp, ctypes.c_size_t, ctypes.c_int,
                                   i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, fp, ctypes.c_int, i64, i64, i64, i64,
                                           ctypes.c_float, ctypes.c_int, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_splitkv_num_splits.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_splitkv_num_splits.restype = ctypes.c_int
    lib.fa_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_qk.argtypes = [vp, vp, vp, vp, fp, vp, ctypes.c_size_t, ctypes.c_int,
                                      i64, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_fwd_splitkv_qk.restype = ctypes.c_int
    lib.fa_splitkv_qk_num_splits.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_splitkv_qk_num_splits.restype = ctypes.c_int
    lib.fa_splitkv_qk_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                  ctypes.c_int]
    lib.fa_splitkv_qk_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_merge_partials.argtypes = [fp, fp, ctypes.c_int, i64, i64, vp, fp, ctypes.c_int, vp]
    lib.fa_merge_partials.restype = ctypes.c_int
    lib.fa_softmax_rows.argtypes = [vp, vp, fp, i64, i64, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.fa_softmax_rows.restype = ctypes.c_int
    lib.fa_softmax_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
    lib.fa_softmax_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_softmax_x_reads.argtypes = [vp, vp, i64, i64, ctypes.c_int]
    lib.fa_softmax_x_reads.restype = ctypes.c_int
    lib.fa_softmax_set_wait_limit.argtypes = [ctypes.c_int]
    lib.fa_softmax_set_wait_limit.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, fp, vp, vp, vp, vp, ctypes.c_size_t,
                           i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_naive_fwd.argtypes = [vp, vp, vp, vp, fp, vp, vp, i64, i64, i64, i64,
                                 ctypes.c_float, ctypes.c_int, vp]
    lib.fa_naive_fwd.restype = ctypes.c_int
    lib.fa_naive_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fa_naive_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------- marshalling

def _device_address(t):
    # Every pointer handed to the library is device memory of the current
    # device (the entry points run under torch.cuda.device of their first
    # tensor): a host tensor or one on another GPU would reach the kernels
    # as an address they cannot use, so it is rejected here.
    if not t.is_cuda:
        raise ValueError(f"tensors must be on a GPU; got one on {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensors must all be on one GPU; got cuda:{t.device.index} "
                         f"alongside cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(_device_address(t))


def _fptr(t):
    return None if t is None else ctypes.cast(ctypes.c_void_p(_device_address(t)),
                                              ctypes.POINTER(ctypes.c_float))


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _shape(q, k, v, o):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be (B, H, N, d), got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return tuple(int(x) for x in q.shape)


def _check(status):
    if status != 0:
        raise FaError(status, fa_last_error())


# --------------------------------------------------------- entry points

def fa_fwd(q, k, v, o, lse, scale, stream=None):
    """Fused forward; writes o (B, H, N, d) and lse (B, H, N) fp32 in place."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, N)):
        raise ValueError("lse must be a contiguous fp32 (B, H, N) tensor")
    with torch.cuda.device(q.device):
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), B, H, N, d,
                        float(scale), _DTYPE_CODE[q.dtype], _stream(stream, q.device))
    _check(st)


_FP8_INPUT = (torch.uint8, torch.float8_e4m3fn)


def fa_fwd_fp8(q, k, v, o, lse, scale, q_scale, k_scale, v_scale, stream=None):
    """FP8 forward: q, k, v are (B, H, N, d) E4M3 codes (uint8 or
    float8_e4m3fn tensors, same shape), o a bf16 tensor of that shape and
    lse a (B, H, N) fp32 tensor, written in place."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype not in _FP8_INPUT:
            raise ValueError(f"{name} must be a contiguous (B, H, N, d) uint8 or "
                             "float8_e4m3fn tensor")
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must match q in shape and device")
    if o.dtype != torch.bfloat16 or o.shape != q.shape or not o.is_contiguous():
        raise ValueError("o must be a contiguous bf16 tensor of q's shape")
    B, H, N, d = (int(x) for x in q.shape)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous fp32 (B, H, N) tensor")
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), B, H, N, d,
                            float(scale), float(q_scale), float(k_scale), float(v_scale),
                            _stream(stream, q.device))
    _check(st)


def fa_fwd_splitkv(q, k, v, o, lse, workspace, scale, num_splits=0, stream=None):
    """Split-KV forward; workspace is a byte (uint8) tensor of at least
    fa_splitkv_workspace_bytes() bytes (may be None when that is 0)."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous fp32 (B, H, N) tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(workspace),
                                ws_bytes, int(num_splits), B, H, N, d, float(scale),
                                _DTYPE_CODE[q.dtype], _stream(stream, q.device))
    _check(st)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, scale, num_splits=0, stream=None):
    """Split-KV forward with its partials in the library's own scratch array
    (FA_NOALLOC_SCRATCH_BYTES per GPU): no workspace argument, nothing
    allocated.  Calls that overlap on one GPU race on that array."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous fp32 (B, H, N) tensor")
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse),
                                        int(num_splits), B, H, N, d, float(scale),
                                        _DTYPE_CODE[q.dtype], _stream(stream, q.device))
    _check(st)


FA_NOALLOC_SCRATCH_BYTES = 64 << 20


def fa_fwd_splitkv_qk(q, k, v, o, lse, workspace, scale, num_splits=0, stream=None):
    """Split-KV forward for queries and keys of different lengths: q and o
    (B, H, Nq, d), k and v (B, H, Nk, d), lse (B, H, Nq) fp32; workspace a
    byte tensor of at least fa_splitkv_qk_workspace_bytes() bytes (may be
    None when that is 0)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D (B, H, N, d) tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, Nq, d = (int(x) for x in q.shape)
    Nk = int(k.shape[2])
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be (B, H, Nk, d) with q's B, H and d")
    if tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("o must have q's shape")
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be a contiguous fp32 (B, H, Nq) tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse),
                                   _ptr(workspace), ws_bytes, int(num_splits), B, H, Nq, Nk, d,
                                   float(scale), _DTYPE_CODE[q.dtype], _stream(stream, q.device))
    _check(st)


def fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, dtype, requested=0):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, code, int(requested)))


def fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, dtype, num_splits=0):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, code,
                                                            int(num_splits)))


def fa_splitkv_num_splits(B, H, N, d, dtype, requested=0):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_splitkv_num_splits(B, H, N, d, code, int(requested)))


def fa_splitkv_workspace_bytes(B, H, N, d, dtype, num_splits=0):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_splitkv_workspace_bytes(B, H, N, d, code, int(num_splits)))


def fa_merge_partials(o_part, lse_part, o, lse, stream=None):
    """Merge partials: o_part (G, rows, d) fp32, lse_part (G, rows) fp32 into
    o (rows, d) and lse (rows) fp32; o's dtype selects the output type."""
    lib = load_library()
    if o_part.dim() != 3 or lse_part.dim() != 2:
        raise ValueError("o_part must be (G, rows, d) and lse_part (G, rows)")
    G, rows, d = (int(x) for x in o_part.shape)
    for name, t, dt in (("o_part", o_part, torch.float32), ("lse_part", lse_part, torch.float32),
                        ("lse", lse, torch.float32)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    if tuple(lse_part.shape) != (G, rows) or tuple(o.shape) != (rows, d) \
            or tuple(lse.shape) != (rows,) or not o.is_contiguous():
        raise ValueError("shapes must be o_part (G, rows, d), lse_part (G, rows), "
                         "o (rows, d), lse (rows,)")
    if o.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {o.dtype}")
    with torch.cuda.device(o.device):
        st = lib.fa_merge_partials(_fptr(o_part), _fptr(lse_part), G, rows, d, _ptr(o),
                                   _fptr(lse), _DTYPE_CODE[o.dtype], _stream(stream, o.device))
    _check(st)


def fa_softmax_rows(x, y, lse=None, workspace=None, stream=None):
    """Row softmax of the 2-D tensor x into y (same shape and dtype; may be
    x itself); lse (rows,) fp32 or None; workspace a byte tensor of at least
    fa_softmax_workspace_bytes() bytes or None when that is 0."""
    lib = load_library()
    if x.dim() != 2 or y.shape != x.shape or y.dtype != x.dtype or not x.is_contiguous() \
            or not y.is_contiguous():
        raise ValueError("x and y must be contiguous 2-D tensors of one shape and dtype")
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {x.dtype}")
    rows, n = (int(t) for t in x.shape)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (rows,)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 (rows,) tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        st = lib.fa_softmax_rows(_ptr(x), _ptr(y), _fptr(lse), rows, n, _DTYPE_CODE[x.dtype],
                                 _ptr(workspace), ws_bytes, _stream(stream, x.device))
    _check(st)


def fa_softmax_workspace_bytes(rows, n, dtype):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_softmax_workspace_bytes(rows, n, code))


def fa_softmax_x_reads(x, y=None):
    """How many times fa_softmax_rows(x, y) would read x from memory on the
    current device (1 or 2); y defaults to x (in place)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    y = x if y is None else y
    return int(load_library().fa_softmax_x_reads(_ptr(x), _ptr(y), x.shape[0], x.shape[1],
                                                 _DTYPE_CODE[x.dtype]))


def fa_softmax_set_wait_limit(polls):
    """Diagnostics: the one-pass softmax's bound on each wait, in polls (0
    sends every slice that finds its row incomplete to the repair kernel;
    negative restores the default).  Returns the previous bound."""
    return int(load_library().fa_softmax_set_wait_limit(int(polls)))


def softmax(x, want_lse=False, stream=None):
    """Allocate y (and lse, workspace) and run fa_softmax_rows on a 2-D x."""
    y = torch.empty_like(x)
    lse = torch.empty(x.shape[0], dtype=torch.float32, device=x.device) if want_lse else None
    nbytes = fa_softmax_workspace_bytes(x.shape[0], x.shape[1], x.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    fa_softmax_rows(x, y, lse, ws, stream)
    return (y, lse) if want_lse else y


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace, scale, stream=None):
    """Backward pass; writes dq, dk, dv in place.  workspace: byte tensor of
    at least fa_bwd_workspace_bytes() bytes."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o)
    for name, t in (("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q in shape and dtype and be contiguous")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 (B, H, N) tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _fptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d, float(scale),
                        _DTYPE_CODE[q.dtype], _stream(stream, q.device))
    _check(st)


def fa_bwd_workspace_bytes(B, H, N):
    return int(load_library().fa_bwd_workspace_bytes(B, H, N))


def backward(q, k, v, o, lse, do, scale=None, stream=None):
    """Allocate dq, dk, dv and the workspace and run the backward pass."""
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa_bwd_workspace_bytes(B, H, N), 16), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale, stream)
    return dq, dk, dv


def fa_naive_fwd(q, k, v, o, lse, s_ws, p_ws, scale, stream=None):
    """Naive three-kernel forward; s_ws and p_ws are byte (uint8) tensors of
    fa_naive_workspace_bytes() bytes each; lse may be None."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o)
    # the softmax kernel writes B*H*N fp32 values through lse when it is given
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, N)):
        raise ValueError("lse must be None or a contiguous fp32 (B, H, N) tensor")
    need = fa_naive_workspace_bytes(B, H, N, q.dtype)
    for name, ws in (("s_ws", s_ws), ("p_ws", p_ws)):
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"{name} holds fewer than {need} bytes")
    with torch.cuda.device(q.device):
        st = lib.fa_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(s_ws),
                              _ptr(p_ws), B, H, N, d, float(scale), _DTYPE_CODE[q.dtype],
                              _stream(stream, q.device))
    _check(st)


def fa_naive_workspace_bytes(B, H, N, dtype):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_naive_workspace_bytes(B, H, N, code))


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def fa_last_error():
    return load_library().fa_last_error().decode()


def fa_version():
    return int(load_library().fa_version())


# ---------------------------------------------------------- conveniences

def default_scale(d):
    """1/sqrt(d) in fp64 rounded once to fp32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def forward(q, k, v, scale=None, stream=None):
    """Allocate O and LSE and run the fused forward.  Returns (o, lse)."""
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, stream)
    return o, lse


def forward_fp8(q, k, v, q_scale, k_scale, v_scale, scale=None, stream=None):
    """Allocate O (bf16) and LSE and run the FP8 forward on E4M3 codes.
    Returns (o, lse)."""
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, o, lse, scale, q_scale, k_scale, v_scale, stream)
    return o, lse


def forward_splitkv(q, k, v, scale=None, num_splits=0, stream=None):
    """Allocate O, LSE and the workspace and run the split-KV forward.
    Returns (o, lse)."""
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    nbytes = fa_splitkv_workspace_bytes(B, H, N, d, q.dtype, num_splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
    fa_fwd_splitkv(q, k, v, o, lse, ws, scale, num_splits, stream)
    return o, lse


def forward_qk(q, k, v, scale=None, num_splits=0, stream=None):
    """Allocate O, LSE and the workspace and run the split-KV forward for q
    (B, H, Nq, d) against k, v (B, H, Nk, d).  Returns (o, lse)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, q.dtype, num_splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
    fa_fwd_splitkv_qk(q, k, v, o, lse, ws, scale, num_splits, stream)
    return o, lse


def naive_forward(q, k, v, scale=None, want_lse=True, stream=None):
    """Allocate O, LSE and both workspaces and run the naive three-kernel
    path.  Returns (o, lse or None)."""
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if want_lse else None
    nbytes = max(fa_naive_workspace_bytes(B, H, N, q.dtype), 16)
    s_ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p_ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_naive_fwd(q, k, v, o, lse, s_ws, p_ws, scale, stream)
    return o, lse
