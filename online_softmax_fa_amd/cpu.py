"""Python binding of libfa_cpu.so, the host-CPU implementation of the same
online-softmax attention forward pass (include/fa_cpu.h).

Argument marshalling only.  This module is separate from the GPU binding:
the GPU entry points never call it, and it never calls them.

  fa_fwd_cpu(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, threads)
  attention_cpu(q, k, v, scale=None, causal=False, kv_len_mask=None, threads=0)
      numpy arrays (float32, or uint16 holding bf16 bits with dtype="bf16")
      -> (o, lse, threads_used)
  cpu_expf(x)
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_cpu.so")
_lib = None


class FaCpuError(RuntimeError):
    def __init__(self, code):
        super().__init__("fa_fwd_cpu error %d" % code)
        self.code = code


def load_library(path=LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FaCpuError(-8)
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd_cpu.restype = ci
    lib.fa_fwd_cpu.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, ci, ci]
    lib.fa_cpu_expf.restype = cf
    lib.fa_cpu_expf.argtypes = [cf]
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.ctypes.data_as(ctypes.c_void_p)


def fa_fwd_cpu(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, threads):
    rc = load_library().fa_fwd_cpu(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N_q, N_k,
                                   d, float(scale), int(bool(causal)), _ptr(kv_len_mask),
                                   int(dtype), int(threads))
    if rc < 0:
        raise FaCpuError(rc)
    return rc


def attention_cpu(q, k, v, scale=None, causal=False, kv_len_mask=None, threads=0, dtype="f32"):
    """q [B,H,Nq,d], k, v [B,H,Nk,d]: contiguous float32 arrays, or uint16
    arrays of bf16 bits with dtype="bf16".  Returns (o, lse, threads_used)."""
    want = np.uint16 if dtype == "bf16" else np.float32
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    for x in (q, k, v):
        if x.dtype != want or x.ndim != 4:
            raise ValueError("q, k, v must be 4-D %s arrays" % np.dtype(want).name)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    m = None if kv_len_mask is None else np.ascontiguousarray(kv_len_mask, dtype=np.uint8)
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float32)
    used = fa_fwd_cpu(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, m,
                      1 if dtype == "bf16" else 0, threads)
    return o, lse, used


def cpu_expf(x):
    return load_library().fa_cpu_expf(float(x))
