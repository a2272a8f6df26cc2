"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
and its Python binding never import, link or call it, and it imports nothing
from them: the two sides share only the seeded input generators.

Contents
  ref_attn.c   the plain definition through a three-pass safe softmax over a
               stored score row, in double (built into ``libfaref.so``)
  online.py    the pages' block-wise online recurrence, in double, for one row
               (block size, traversal order and a per-block trace are inputs)

Public functions
  build()                       compile ``libfaref.so`` with gcc
  attn_fwd(q, k, v, ...)        o, lse for all or selected query rows
  softmax_row(s, vis)           p, m, l for one precomputed score row
  attn_from_scores(s, v, vis)   o, lse for one precomputed score row
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref_attn.c")
_LIB = os.path.join(_HERE, "libfaref.so")
_lib = None


def build(force=True):
    """Compile the C oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, dbl = ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.ref_softmax_weighted_sum.restype = i64
    lib.ref_softmax_weighted_sum.argtypes = [vp, vp, i64, vp, i64, i64, vp, vp, vp, vp, vp]
    lib.ref_attn_rows.restype = ctypes.c_int
    lib.ref_attn_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, dbl, ctypes.c_int,
                                  vp, vp, i64, vp, vp, ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_f32(x, name):
    a = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    if a.ndim != 4:
        raise ValueError("%s must be [B, H, N, d]" % name)
    return a


def attn_fwd(q, k, v, scale, causal=False, mask=None, rows=None, threads=0):
    """Attention forward in fp64.

    q [B,H,Nq,d], k and v [B,H,Nk,d]: fp32 arrays (bf16 data widened to fp32
    beforehand, which is exact).  scale is rounded to float32, as the library
    receives it, and that value is used in double.  mask: None or uint8/bool
    [B, Nk], nonzero = visible.  rows: None for every row (returns o [B,H,Nq,d], lse [B,H,Nq]),
    or a 1-D array of flat row indices (b*H + h)*Nq + i (returns o [n, d],
    lse [n]).  Returns (o, lse, threads_used).
    """
    q, k, v = _as_f32(q, "q"), _as_f32(k, "k"), _as_f32(v, "v")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d):
        raise ValueError("k, v must be [B, H, Nk, d] matching q")
    m = None
    if mask is not None:
        m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        if m.shape != (B, Nk):
            raise ValueError("mask must be [B, Nk]")
    r = None
    nrows = B * H * Nq
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows), dtype=np.int64).ravel()
        nrows = r.shape[0]
    o = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    used = _load().ref_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, d,
                                 float(np.float32(scale)), int(bool(causal)), _ptr(m), _ptr(r),
                                 nrows, _ptr(o), _ptr(lse), int(threads))
    if used < 0:
        raise RuntimeError("ref_attn_rows failed with code %d" % used)
    if rows is None:
        o = o.reshape(B, H, Nq, d)
        lse = lse.reshape(B, H, Nq)
    return o, lse, used


def _row_args(s, vis):
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64).ravel())
    vv = None
    if vis is not None:
        vv = np.ascontiguousarray(np.asarray(vis) != 0, dtype=np.uint8).ravel()
        if vv.shape != s.shape:
            raise ValueError("vis must match the score row")
    return s, vv


def softmax_row(s, vis=None):
    """Three-pass safe softmax of one score row: returns (p, m, l)."""
    s, vv = _row_args(s, vis)
    n = s.shape[0]
    p = np.empty(n, dtype=np.float64)
    o = np.empty(1, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    m = ctypes.c_double()
    l = ctypes.c_double()
    _load().ref_softmax_weighted_sum(_ptr(s), _ptr(vv), n, None, 0, 0, _ptr(o), _ptr(lse),
                                     _ptr(p), ctypes.byref(m), ctypes.byref(l))
    return p, m.value, l.value


def attn_from_scores(s, v, vis=None):
    """Softmax-weighted sum of value rows for one score row: returns (o, lse).

    v is n x dv; its entries are taken as fp32 (the toy examples' values are
    exact in fp32).
    """
    s, vv = _row_args(s, vis)
    n = s.shape[0]
    va = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(n, -1))
    dv = va.shape[1]
    o = np.empty(dv, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    _load().ref_softmax_weighted_sum(_ptr(s), _ptr(vv), n, _ptr(va), dv, dv, _ptr(o),
                                     _ptr(lse), None, None, None)
    return o, float(lse[0])
