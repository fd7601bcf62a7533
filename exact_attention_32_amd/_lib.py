"""ctypes binding of libfa (include/fa.h): forward, backward and decode.  Argument marshalling only: every
step of the computation runs in the HIP kernels of the library.

There is no fallback: if ``libfa.so`` has not been built, or cannot be
loaded, every entry point raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")
# The checking build (FA_SAFE_SYNC=1: every LDS copy completed at a barrier
# before use); only the tests load it.
SAFE_SYNC_LIB_PATH = os.path.join(HERE, "libfa_safesync.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_SCALE = 4
FA_ERR_ALIGN = 5
FA_ERR_HIP = 6
FA_ERR_ALIAS = 7
FA_ERR_WORKSPACE = 8
FA_ERR_DTYPE = 9
FA_ERR_STRIDE = 10
FA_ERR_SCRATCH = 11
# bytes of the fixed device scratch of fa_decode_noalloc (include/fa.h)
FA_DECODE_SCRATCH_BYTES = 17 << 20
FA_DTYPE_BF16 = 0
FA_DTYPE_FP16 = 1

EXPORTS = ("fa_bwd", "fa_bwd_ex", "fa_decode", "fa_decode_ex", "fa_decode_noalloc",
           "fa_decode_workspace_size",
           "fa_fwd", "fa_fwd_ex", "fa_fwd_f32", "fa_fwd_kv_outer", "fa_fwd_kv_outer_workspace_size",
           "fa_strerror")

_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A fresh handle on a build of the library at ``path`` (e.g. the checking
    build libfa_safesync.so) with the C ABI's argument types declared."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m exact_attention_32_amd.build_lib` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(lib, name)
        fn.restype = i
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [i] + [vp] * 10 + [i, i, i, i, f, i, ctypes.POINTER(ctypes.c_int64),
                                                 vp]
    lib.fa_decode.restype = i
    lib.fa_decode.argtypes = [vp] * 5 + [i] * 5 + [f, i, i, vp, ctypes.c_size_t, vp]
    lib.fa_decode_ex.restype = i
    lib.fa_decode_ex.argtypes = ([i] + [vp] * 5 + [i] * 5 + [f, i, i, vp, ctypes.c_size_t,
                                                             ctypes.POINTER(ctypes.c_int64), vp])
    lib.fa_decode_noalloc.restype = i
    lib.fa_decode_noalloc.argtypes = [vp] * 5 + [i] * 5 + [f, i, i, vp]
    lib.fa_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_decode_workspace_size.argtypes = [i] * 6
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_ex.argtypes = [i] + [vp] * 5 + [i] * 4 + [f, i, ctypes.POINTER(ctypes.c_int64), vp]
    lib.fa_fwd_kv_outer.restype = i
    lib.fa_fwd_kv_outer.argtypes = [vp] * 5 + [i] * 4 + [f, i, vp, ctypes.c_size_t, vp]
    lib.fa_fwd_kv_outer_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_kv_outer_workspace_size.argtypes = [i] * 4
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [i]
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int | None:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def _resolve_stream(stream, device):
    """The torch stream the work goes to: ``stream`` itself (a torch stream, or
    a raw HIP stream handle wrapped as an external stream), else the current
    stream of ``device``.  Buffers the wrappers allocate are allocated while
    this stream is current, so the caching allocator hands their memory to
    later allocations on other streams only after this stream's work."""
    import torch

    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _check_out(t, name, shape, dtype, dense=False):
    """Reject a caller-supplied output the kernels could not write safely:
    the C ABI sees only its address, so its shape, type, device and layout
    are checked here; the callers check its device afterwards."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not dense and t.dim() == 4 and t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")


def fa_strerror(code: int) -> str:
    return load_library().fa_strerror(int(code)).decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """Enqueue the bf16 forward pass; pointers may be ints or tensors.
    Returns the fa_status code (0 on success)."""
    return int(load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     int(B), int(H), int(N), int(d), float(scale),
                                     int(bool(causal)), _stream(stream)))


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """Enqueue the fp32 forward pass; same arguments as fa_fwd."""
    return int(load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         int(B), int(H), int(N), int(d), float(scale),
                                         int(bool(causal)), _stream(stream)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal,
           stream=None) -> int:
    """Enqueue the bf16 backward pass; pointers may be ints or tensors.
    Returns the fa_status code (0 on success)."""
    return int(load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                     _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                     int(B), int(H), int(N), int(d), float(scale),
                                     int(bool(causal)), _stream(stream)))


def fa_bwd_ex(dtype, q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, strides,
              stream=None) -> int:
    """Enqueue the backward pass on bf16 or fp16 strided views.  ``strides``
    is a sequence of 24 element strides (q, k, v, o, dout, dq, dk, dv: batch,
    head, row), or None for a NULL pointer.  Returns the fa_status code."""
    arr = None
    if strides is not None:
        arr = (ctypes.c_int64 * 24)(*[int(x) for x in strides])
    return int(load_library().fa_bwd_ex(int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                        _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                        int(B), int(H), int(N), int(d), float(scale),
                                        int(bool(causal)), arr, _stream(stream)))


def fa_fwd_ex(dtype, q, k, v, o, lse, B, H, N, d, scale, causal, strides, stream=None) -> int:
    """Enqueue the forward pass on bf16 or fp16 strided views.  ``strides``
    is a sequence of 12 element strides (q, k, v, o: batch, head, row), or
    None for a NULL pointer.  Returns the fa_status code."""
    arr = None
    if strides is not None:
        arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides])
    return int(load_library().fa_fwd_ex(int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        int(B), int(H), int(N), int(d), float(scale),
                                        int(bool(causal)), arr, _stream(stream)))


def fa_fwd_kv_outer(q, k, v, o, lse, B, H, N, d, scale, causal, workspace, workspace_bytes,
                    stream=None) -> int:
    """Enqueue the key/value-outer (Algorithm 1 order) forward pass; pointers
    may be ints or tensors.  Returns the fa_status code."""
    return int(load_library().fa_fwd_kv_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              int(B), int(H), int(N), int(d), float(scale),
                                              int(bool(causal)), _ptr(workspace),
                                              int(workspace_bytes), _stream(stream)))


def fa_fwd_kv_outer_workspace_size(B, H, N, d) -> int:
    return int(load_library().fa_fwd_kv_outer_workspace_size(int(B), int(H), int(N), int(d)))


def fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, workspace,
              workspace_bytes, stream=None) -> int:
    """Enqueue the decode kernels; pointers may be ints or tensors.  Returns
    the fa_status code (0 on success)."""
    return int(load_library().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
                                        int(bool(causal)), int(num_splits), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream)))


def fa_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits,
                      stream=None) -> int:
    """Enqueue fa_decode with the library's fixed scratch instead of a
    workspace (nothing is allocated).  Returns the fa_status code
    (FA_ERR_SCRATCH when the partials exceed FA_DECODE_SCRATCH_BYTES)."""
    return int(load_library().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                int(B), int(H), int(Nq), int(Nk), int(d),
                                                float(scale), int(bool(causal)), int(num_splits),
                                                _stream(stream)))


def fa_decode_ex(dtype, q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, workspace,
                 workspace_bytes, strides, stream=None) -> int:
    """Enqueue the decode pass on bf16 or fp16 strided views.  ``strides`` is
    a sequence of 12 element strides (q, k, v, o: batch, head, row), or None
    for a NULL pointer.  Returns the fa_status code."""
    arr = None
    if strides is not None:
        arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides])
    return int(load_library().fa_decode_ex(int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                           _ptr(lse), int(B), int(H), int(Nq), int(Nk), int(d),
                                           float(scale), int(bool(causal)), int(num_splits),
                                           _ptr(workspace), int(workspace_bytes), arr,
                                           _stream(stream)))


def fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits=0) -> int:
    return int(load_library().fa_decode_workspace_size(int(B), int(H), int(Nq), int(Nk),
                                                       int(d), int(num_splits)))


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            stream=None):
    """Torch convenience wrapper: q, k, v are [B, H, N, d] device tensors, all
    bf16, all fp16 or all fp32.  bf16 and fp16 may be strided views whose last
    dimension is contiguous (fa_fwd_ex; dense bf16 goes to fa_fwd); fp32 must
    be contiguous (fa_fwd_f32).  Allocates O (input dtype, dense) and LSE
    (fp32, [B, H, N]) unless given, enqueues the kernel on ``stream``
    (default: the current torch stream) and returns (O, LSE).  ``scale``
    defaults to 1/sqrt(d), the factor of the attention definition."""
    import torch

    if not (q.shape == k.shape == v.shape and q.dim() == 4):
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16,
                                                             torch.float32):
        raise TypeError("q, k, v must all be bfloat16, all float16 or all float32")
    B, H, N, d = q.shape
    if out is not None:
        _check_out(out, "out", q.shape, q.dtype, dense=q.dtype == torch.float32)
    if lse is not None:
        _check_out(lse, "lse", (B, H, N), torch.float32, dense=True)
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one device")
    for t, name in ((out, "out"), (lse, "lse")):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, got {t.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _resolve_stream(stream, q.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dense = all(t.is_contiguous() for t in (q, k, v, out))
    if q.dtype == torch.float32:
        if not dense:
            raise ValueError("float32 tensors must be contiguous")
        rc = fa_fwd_f32(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
    elif q.dtype == torch.bfloat16 and dense:
        rc = fa_fwd(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
    else:
        if any(t.stride(3) != 1 for t in (q, k, v, out)):
            raise ValueError("the last dimension must be contiguous")
        strides = [x for t in (q, k, v, out) for x in t.stride()[:3]]
        dt = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
        rc = fa_fwd_ex(dt, q, k, v, out, lse, B, H, N, d, scale, causal, strides, stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             stream=None, out=None):
    """Torch convenience wrapper of the backward pass: q, k, v, o, dout are
    [B, H, N, d] device tensors, all bf16 or all fp16, and (o, lse) what
    ``forward`` returned for q, k, v with the same causal and scale.  Dense
    bf16 goes to fa_bwd; fp16 or strided views (last dimension contiguous) to
    fa_bwd_ex.  Allocates dQ, dK, dV (dense, the input dtype) unless ``out``
    gives them, and the fp32 [B, H, N] workspace delta; enqueues the two
    kernels on ``stream`` (default: the current torch stream) and returns
    (dQ, dK, dV, delta)."""
    import torch

    ts = (q, k, v, o, dout)
    if not (all(t.shape == q.shape for t in ts) and q.dim() == 4):
        raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape")
    if not all(t.dtype == q.dtype for t in ts) or q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q, k, v, o, dout must all be bfloat16 or all float16")
    B, H, N, d = q.shape
    _check_out(lse, "lse", (B, H, N), torch.float32, dense=True)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a (dq, dk, dv) triple")
        for t, name in zip(out, ("dq", "dk", "dv")):
            _check_out(t, name, q.shape, q.dtype)
    if not all(t.is_cuda for t in ts + (lse,)):
        raise ValueError("all tensors must be device tensors")
    for t in ts[1:] + (lse,) + (tuple(out) if out is not None else ()):
        if t.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, got {t.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _resolve_stream(stream, q.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = tuple(torch.empty(q.shape, dtype=q.dtype, device=q.device) for _ in range(3))
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = out
    tensors = ts + (dq, dk, dv)
    if q.dtype == torch.bfloat16 and all(t.is_contiguous() for t in tensors):
        rc = fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)
    else:
        if any(t.stride(3) != 1 for t in tensors):
            raise ValueError("the last dimension must be contiguous")
        strides = [x for t in tensors for x in t.stride()[:3]]
        dt = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
        rc = fa_bwd_ex(dt, q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal,
                       strides, stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return dq, dk, dv, delta


def decode(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0,
           stream=None, out=None):
    """Torch convenience wrapper of the decode pass: q is a [B, H, Nq, d]
    device tensor (Nq <= 16), k and v [B, H, Nk, d], all bf16 or all fp16.
    Dense bf16 goes to fa_decode; fp16 or strided views (last dimension
    contiguous; e.g. a [B, Nk, H, d] key/value cache) to fa_decode_ex.
    Allocates O (dense, the input dtype) unless ``out`` gives it, LSE and the
    workspace, enqueues the kernels on ``stream`` (default: the current torch
    stream) and returns (O, LSE)."""
    import torch

    if not (q.dim() == k.dim() == 4 and k.shape == v.shape and q.shape[:2] == k.shape[:2]
            and q.shape[3] == k.shape[3]):
        raise ValueError("need q [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q, k, v must all be bfloat16 or all float16")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if out is not None:
        _check_out(out, "out", q.shape, q.dtype)
    if not all(t.is_cuda for t in (q, k, v)):
        raise ValueError("q, k, v must be device tensors")
    for t in (k, v) + ((out,) if out is not None else ()):
        if t.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, got {t.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits)
    if need == 0:
        raise FAError(FA_ERR_SHAPE, fa_strerror(FA_ERR_SHAPE))
    stream = _resolve_stream(stream, q.device)
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device) if out is None else out
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    tensors = (q, k, v, o)
    if q.dtype == torch.bfloat16 and all(t.is_contiguous() for t in tensors):
        rc = fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, ws, need,
                       stream)
    else:
        if any(t.stride(3) != 1 for t in tensors):
            raise ValueError("the last dimension must be contiguous")
        strides = [x for t in tensors for x in t.stride()[:3]]
        dt = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
        rc = fa_decode_ex(dt, q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits, ws,
                          need, strides, stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return o, lse


def forward_kv_outer(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Torch convenience wrapper of fa_fwd_kv_outer (bf16 [B, H, N, d] device
    tensors): allocates O, LSE and the fp32 state workspace, returns (O, LSE)."""
    import torch

    if not (q.shape == k.shape == v.shape and q.dim() == 4):
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)):
        raise TypeError("q, k, v must be bfloat16")
    if not all(t.is_cuda and t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must be contiguous device tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fwd_kv_outer_workspace_size(B, H, N, d)
    if need == 0:
        raise FAError(FA_ERR_SHAPE, fa_strerror(FA_ERR_SHAPE))
    stream = _resolve_stream(stream, q.device)
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = fa_fwd_kv_outer(q, k, v, o, lse, B, H, N, d, scale, causal, ws, need, stream)
    if rc != FA_OK:
        raise FAError(rc, fa_strerror(rc))
    return o, lse
