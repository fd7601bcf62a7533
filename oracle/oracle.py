"""ctypes front end of the fp64 CPU oracle in ``oracle.c`` (forward pass and
its gradients).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never imports it.

The oracle is the plain definition of attention (page "解析 FlashAttention（2）",
sections 1.1, 2.1 eq. (2)-(5) and 3.2; causal masking from the causal-mask
lesson of "在线 Softmax 与 FlashAttention").  All arithmetic happens in C in
fp64; this file only converts arrays and checks shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -O2 without any fast-math flag: IEEE semantics, exp/log from libm.
CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Wextra"]

_lock = threading.Lock()
_default = None


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile ``src`` with gcc into the shared library ``out``; returns ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.POINTER(ctypes.c_long)


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _as_f64(x) -> np.ndarray:
    """Widen any real array (numpy, or a CPU torch tensor in fp32/bf16/fp64) to
    a C-contiguous float64 numpy array.  Widening fp32 and bf16 to fp64 is
    exact."""
    if hasattr(x, "detach"):  # torch tensor: go through fp32 (exact for bf16)
        import torch

        t = x.detach().to("cpu")
        if t.dtype != torch.float64:
            t = t.to(torch.float32)
        x = t.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


class Oracle:
    """One loaded copy of the oracle library (tests may load a planted-mistake
    build of the same source under another path)."""

    def __init__(self, libpath: str = LIB):
        self.libpath = libpath
        lib = ctypes.CDLL(libpath)
        lib.oracle_softmax.restype = ctypes.c_double
        lib.oracle_softmax.argtypes = [_D, ctypes.c_long, _D]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [_D, _D, _D] + [ctypes.c_long] * 4 + [
            ctypes.c_double, ctypes.c_int, _D, _D]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [_D, _D, _D] + [ctypes.c_long] * 4 + [
            ctypes.c_double, ctypes.c_int, _L, ctypes.c_long, _D, _D]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [_D, _D, _D, _D] + [ctypes.c_long] * 4 + [
            ctypes.c_double, ctypes.c_int, _D, _D, _D]
        lib.oracle_attention_backward_dq_rows.restype = ctypes.c_int
        lib.oracle_attention_backward_dq_rows.argtypes = [_D, _D, _D, _D] + [ctypes.c_long] * 4 + [
            ctypes.c_double, ctypes.c_int, _L, ctypes.c_long, _D]
        lib.oracle_attention_backward_kv_keys.restype = ctypes.c_int
        lib.oracle_attention_backward_kv_keys.argtypes = [_D, _D, _D, _D, ctypes.c_long,
                                                          ctypes.c_long, ctypes.c_double,
                                                          ctypes.c_int, _L, ctypes.c_long, _D, _D]
        lib.oracle_attention_qk.restype = ctypes.c_int
        lib.oracle_attention_qk.argtypes = [_D, _D, _D] + [ctypes.c_long] * 5 + [
            ctypes.c_double, ctypes.c_int, _D, _D]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        self._lib = lib

    # -- safe softmax of one vector (eq. (2)-(5)) --------------------------
    def softmax(self, x):
        """Returns (p, lse) for a 1-D vector; -inf entries are masked."""
        x = _as_f64(x).reshape(-1)
        p = np.empty_like(x)
        lse = self._lib.oracle_softmax(_dptr(x), x.size, _dptr(p))
        return p, lse

    # -- full forward ------------------------------------------------------
    def attention(self, q, k, v, scale: float, causal: bool):
        """q, k, v: [B, H, N, d] (or [N, d]).  Returns (O [B,H,N,d], LSE [B,H,N])
        in float64.  ``scale`` is used exactly as given (pass the fp32 value
        the GPU receives, widened)."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        squeeze = q.ndim == 2
        if squeeze:
            q, k, v = q[None, None], k[None, None], v[None, None]
        if not (q.shape == k.shape == v.shape and q.ndim == 4):
            raise ValueError("q, k, v must share one [B,H,N,d] shape")
        B, H, N, d = q.shape
        o = np.empty_like(q)
        lse = np.empty((B, H, N), dtype=np.float64)
        rc = self._lib.oracle_attention(_dptr(q), _dptr(k), _dptr(v), B, H, N, d,
                                        float(scale), int(bool(causal)),
                                        _dptr(o), _dptr(lse))
        if rc != 0:
            raise MemoryError("oracle_attention: out of memory for S")
        if squeeze:
            return o[0, 0], lse[0, 0]
        return o, lse

    # -- queries and keys of different lengths (decode) ---------------------
    def attention_qk(self, q, k, v, scale: float, causal: bool):
        """q: [B, H, Nq, d]; k, v: [B, H, Nk, d] with Nq <= Nk.  The queries are
        the last Nq positions (causal: query i sees keys j <= Nk - Nq + i).
        Returns (O [B, H, Nq, d], LSE [B, H, Nq]) in float64."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        if not (q.ndim == k.ndim == 4 and k.shape == v.shape and q.shape[:2] == k.shape[:2]
                and q.shape[3] == k.shape[3] and q.shape[2] <= k.shape[2]):
            raise ValueError("need q [B,H,Nq,d], k and v [B,H,Nk,d], Nq <= Nk")
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        o = np.empty_like(q)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self._lib.oracle_attention_qk(_dptr(q), _dptr(k), _dptr(v), B, H, Nq, Nk, d,
                                           float(scale), int(bool(causal)), _dptr(o), _dptr(lse))
        if rc != 0:
            raise ValueError("oracle_attention_qk: bad shape or out of memory")
        return o, lse

    # -- selected rows only --------------------------------------------------
    def attention_rows(self, q, k, v, scale: float, causal: bool, rows):
        """rows: int array [R, 3] of (b, h, i).  Returns (O_rows [R, d],
        LSE_rows [R]) computed from the definition for those rows only."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        if not (q.shape == k.shape == v.shape and q.ndim == 4):
            raise ValueError("q, k, v must share one [B,H,N,d] shape")
        B, H, N, d = q.shape
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        o = np.empty((r.shape[0], d), dtype=np.float64)
        lse = np.empty((r.shape[0],), dtype=np.float64)
        rc = self._lib.oracle_attention_rows(
            _dptr(q), _dptr(k), _dptr(v), B, H, N, d, float(scale),
            int(bool(causal)), r.ctypes.data_as(_L), r.shape[0], _dptr(o), _dptr(lse))
        if rc != 0:
            raise ValueError("oracle_attention_rows: bad row index or out of memory")
        return o, lse

    # -- backward (gradients of the forward definition) ----------------------
    def attention_backward(self, q, k, v, dout, scale: float, causal: bool):
        """q, k, v, dout: [B, H, N, d] (or [N, d]).  Returns (dQ, dK, dV) of
        the forward definition for the output gradient ``dout``, in float64."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        squeeze = q.ndim == 2
        if squeeze:
            q, k, v, dout = q[None, None], k[None, None], v[None, None], dout[None, None]
        if not (q.shape == k.shape == v.shape == dout.shape and q.ndim == 4):
            raise ValueError("q, k, v, dout must share one [B,H,N,d] shape")
        B, H, N, d = q.shape
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        rc = self._lib.oracle_attention_backward(
            _dptr(q), _dptr(k), _dptr(v), _dptr(dout), B, H, N, d, float(scale),
            int(bool(causal)), _dptr(dq), _dptr(dk), _dptr(dv))
        if rc != 0:
            raise MemoryError("oracle_attention_backward: out of memory")
        if squeeze:
            return dq[0, 0], dk[0, 0], dv[0, 0]
        return dq, dk, dv

    def attention_backward_dq_rows(self, q, k, v, dout, scale: float, causal: bool, rows):
        """rows: int array [R, 3] of (b, h, i).  Returns dQ rows [R, d]."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        if not (q.shape == k.shape == v.shape == dout.shape and q.ndim == 4):
            raise ValueError("q, k, v, dout must share one [B,H,N,d] shape")
        B, H, N, d = q.shape
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.empty((r.shape[0], d), dtype=np.float64)
        rc = self._lib.oracle_attention_backward_dq_rows(
            _dptr(q), _dptr(k), _dptr(v), _dptr(dout), B, H, N, d, float(scale),
            int(bool(causal)), r.ctypes.data_as(_L), r.shape[0], _dptr(out))
        if rc != 0:
            raise ValueError("oracle_attention_backward_dq_rows: bad row index or out of memory")
        return out

    def attention_backward_kv_keys(self, q, k, v, dout, scale: float, causal: bool, keys):
        """One head: q, k, v, dout are [N, d].  Returns (dK rows, dV rows),
        each [len(keys), d], for the given key indices."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        if not (q.shape == k.shape == v.shape == dout.shape and q.ndim == 2):
            raise ValueError("q, k, v, dout must share one [N, d] shape")
        N, d = q.shape
        kk = np.ascontiguousarray(np.asarray(keys, dtype=np.int64).reshape(-1))
        dk = np.empty((kk.size, d), dtype=np.float64)
        dv = np.empty((kk.size, d), dtype=np.float64)
        rc = self._lib.oracle_attention_backward_kv_keys(
            _dptr(q), _dptr(k), _dptr(v), _dptr(dout), N, d, float(scale), int(bool(causal)),
            kk.ctypes.data_as(_L), kk.size, _dptr(dk), _dptr(dv))
        if rc != 0:
            raise ValueError("oracle_attention_backward_kv_keys: bad key or out of memory")
        return dk, dv

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self._lib.oracle_set_num_threads(int(n))


def default() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory (built on first use
    if no library is there yet)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB):
                build()
            _default = Oracle(LIB)
        return _default
