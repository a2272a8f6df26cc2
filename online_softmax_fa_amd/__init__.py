"""Python binding of libfa.so, the gfx950 exact attention forward pass.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa.so``; this module turns torch tensors into device pointers
and sizes, passes torch's current HIP stream, and raises on a non-zero status.
There is no fallback: if the library is missing or fails to load, every call
raises.

Entry points (same names and meaning as include/fa.h):
  fa_fwd(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, stream)
  fa_fwd_ex(..., opts)
  fa_strerror(code)
and one convenience wrapper that allocates the outputs with torch:
  attention(q, k, v, scale=None, causal=False, kv_len_mask=None, block_n=0, reverse_kv=False)
      -> (o, lse)
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEAD_DIM = -3
FA_ERR_DTYPE = -4
FA_ERR_SCALE = -5
FA_ERR_TILE = -6
FA_ERR_DEVICE = -7
FA_ERR_LAUNCH = -8
FA_ERR_ALIAS = -9

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1


class FaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("fa error %d: %s" % (code, msg))
        self.code = code


class fa_opts(ctypes.Structure):
    _fields_ = [("block_n", ctypes.c_int), ("reverse_kv", ctypes.c_int)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libfa.so (once).  torch is imported first so that the process has
    exactly one HIP runtime: torch's, which libfa.so then binds to."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime libfa.so will use)
    if not os.path.exists(path):
        raise FaError(FA_ERR_LAUNCH, "libfa.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    args = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_fwd.argtypes = args
    lib.fa_fwd_ex.restype = ci
    lib.fa_fwd_ex.argtypes = args + [ctypes.POINTER(fa_opts)]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [ci]
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def fa_strerror(code):
    return load_library().fa_strerror(int(code)).decode()


def _check(rc):
    if rc != FA_OK:
        raise FaError(rc, fa_strerror(rc))


def fa_fwd(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, stream):
    """C fa_fwd.  Tensors or raw device addresses; stream is a hipStream_t
    handle (int) or None for the default stream."""
    rc = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N_q, N_k, d,
                               float(scale), int(bool(causal)), _ptr(kv_len_mask), int(dtype),
                               stream)
    _check(rc)


def fa_fwd_ex(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, stream,
              opts=None):
    """C fa_fwd_ex; opts is an fa_opts or None."""
    rc = load_library().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N_q, N_k,
                                  d, float(scale), int(bool(causal)), _ptr(kv_len_mask),
                                  int(dtype), stream,
                                  ctypes.byref(opts) if opts is not None else None)
    _check(rc)


def attention(q, k, v, scale=None, causal=False, kv_len_mask=None, block_n=0, reverse_kv=False,
              out=None):
    """o, lse for torch tensors q [B,H,Nq,d], k, v [B,H,Nk,d] on one GPU.

    q, k, v: contiguous float32 or bfloat16 CUDA (HIP) tensors; kv_len_mask:
    None or a uint8 [B, Nk] CUDA tensor.  Outputs are allocated with torch
    (o in the input dtype, lse float32) unless `out=(o, lse)` is given.  The
    kernel runs on torch's current stream; nothing is synchronised.
    """
    import torch
    if q.dtype == torch.bfloat16:
        dt = FA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = FA_DTYPE_F32
    else:
        raise FaError(FA_ERR_DTYPE, "q must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise FaError(FA_ERR_SHAPE, "%s must be a contiguous 4-D GPU tensor of q's dtype" % name)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise FaError(FA_ERR_SHAPE, "k and v must be [B, H, N_k, d] matching q")
    if kv_len_mask is not None:
        if (kv_len_mask.dtype != torch.uint8 or not kv_len_mask.is_cuda
                or not kv_len_mask.is_contiguous() or tuple(kv_len_mask.shape) != (B, Nk)):
            raise FaError(FA_ERR_SHAPE, "kv_len_mask must be a contiguous uint8 [B, N_k] GPU tensor")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = fa_opts(int(block_n), int(bool(reverse_kv)))
    fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_len_mask, dt, stream, opts)
    return o, lse
