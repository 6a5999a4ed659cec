"""Python binding of ``libattn_cpu.so``: the cache-blocked multi-core CPU form
of the same fused, exact attention (``include/attn_cpu.h``).

Host numpy arrays, float32 [B, H, N, d]; the binding only marshals arguments
(every step runs in the C++ library).  This is an implementation for CPUs in
its own right, not a fallback of the GPU path: nothing in the GPU binding
calls it.  If the library is missing, loading it raises.

* :func:`attn_cpu_fwd` (q, k, v, causal, scale, threads) -> (o, lse)
* :func:`attn_cpu_bwd` (q, k, v, o, do, lse, causal, scale, threads) -> (dq, dk, dv)
"""

import ctypes
import math
import os

import numpy as np

__all__ = ["attn_cpu_fwd", "attn_cpu_bwd", "lib", "CPU_LIB_PATH"]

CPU_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_cpu.so")
_lib = None


def lib():
    """The loaded ``libattn_cpu.so`` (raises OSError if it was not built)."""
    global _lib
    if _lib is None:
        L = ctypes.CDLL(CPU_LIB_PATH)
        fp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.attn_cpu_fwd.argtypes = [fp] * 5 + [i64] * 4 + [i32, f32, i32]
        L.attn_cpu_fwd.restype = i32
        L.attn_cpu_bwd.argtypes = [fp] * 9 + [i64] * 4 + [i32, f32, i32]
        L.attn_cpu_bwd.restype = i32
        _lib = L
    return _lib


def _f32(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 4:
        raise ValueError("expected a [B, H, N, d] array")
    return x


def _ptr(x):
    return x.ctypes.data_as(ctypes.c_void_p)


def _check(status, where):
    if status != 0:
        raise RuntimeError(f"{where}: status {status}")


def attn_cpu_fwd(q, k, v, causal=False, scale=None, threads=0):
    q, k, v = _f32(q), _f32(k), _f32(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float32)
    st = lib().attn_cpu_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), scale,
                            int(threads))
    _check(st, "attn_cpu_fwd")
    return o, lse


def attn_cpu_bwd(q, k, v, o, do, lse, causal=False, scale=None, threads=0):
    q, k, v, o, do = (_f32(x) for x in (q, k, v, o, do))
    lse = np.ascontiguousarray(lse, dtype=np.float32)
    B, H, N, d = q.shape
    if not (k.shape == v.shape == o.shape == do.shape == q.shape) or lse.shape != (B, H, N):
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    st = lib().attn_cpu_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B,
                            H, N, d, int(bool(causal)), scale, int(threads))
    _check(st, "attn_cpu_bwd")
    return dq, dk, dv
