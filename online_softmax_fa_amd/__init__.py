"""Python binding of libfa.so, the gfx950 exact attention forward pass.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa.so``; this module turns torch tensors into device pointers
and sizes, passes torch's current HIP stream, and raises on a non-zero status.
There is no fallback: if the library is missing or fails to load, every call
raises.

Entry points (same names and meaning as include/fa.h):
  fa_fwd(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype, stream)
  fa_fwd_ex(..., opts)
  fa_splitkv_workspace_bytes(B, H, N_q, d, num_splits)
  fa_splitkv_splits(B, H, N_q, N_k, d, causal)
  fa_fwd_splitkv(..., dtype, num_splits, workspace, workspace_bytes, stream)
  fa_fwd_splitkv_noalloc(..., dtype, num_splits, stream)
  fa_merge_states(m, l, acc, n_parts, rows, d, scale, o, lse, dtype, stream)
  fa_softmax_rows(s, p, m, l, rows, n, dtype, stream)
  fa_strerror(code)
and convenience wrappers that allocate outputs (and workspace) with torch:
  attention(q, k, v, scale=None, causal=False, kv_len_mask=None, block_n=0, reverse_kv=False,
            out=None, trace=None)                                   -> (o, lse)
  attention_splitkv(q, k, v, scale=None, causal=False, kv_len_mask=None, num_splits=None,
                    out=None, workspace=None)                       -> (o, lse)
  merge_states(m, l, acc, scale, out_dtype=None, out=None)          -> (o, lse)
  softmax_rows(s, out=None)                                         -> (p, m, l)
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
FA_ERR_ARG = -10
FA_ERR_WORKSPACE = -11
FA_ERR_ALIGN = -12
FA_ERR_SCRATCH = -13

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1


class FaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("fa error %d: %s" % (code, msg))
        self.code = code


class fa_opts(ctypes.Structure):
    _fields_ = [("block_n", ctypes.c_int), ("reverse_kv", ctypes.c_int),
                ("trace", ctypes.c_void_p), ("trace_b", ctypes.c_int), ("trace_h", ctypes.c_int),
                ("trace_row", ctypes.c_int)]


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
    sz, i64 = ctypes.c_size_t, ctypes.c_int64
    lib.fa_splitkv_workspace_bytes.restype = sz
    lib.fa_splitkv_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.fa_splitkv_splits.restype = ci
    lib.fa_splitkv_splits.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.fa_fwd_splitkv.restype = ci
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, ci, ci, vp,
                                   sz, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ci
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, ci,
                                           ci, vp]
    lib.fa_merge_states.restype = ci
    lib.fa_merge_states.argtypes = [vp, vp, vp, ci, i64, ci, cf, vp, vp, ci, vp]
    lib.fa_softmax_rows.restype = ci
    lib.fa_softmax_rows.argtypes = [vp, vp, vp, vp, i64, i64, ci, vp]
    lib.fa_query_tile_rows.restype = ci
    lib.fa_query_tile_rows.argtypes = [ci, ci, ci, ci, ci, ci, ci]
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


def fa_query_tile_rows(dtype, B, H, N_q, d, block_n=0, causal=False):
    """C fa_query_tile_rows: query rows per workgroup of fa_fwd."""
    rc = load_library().fa_query_tile_rows(int(dtype), int(B), int(H), int(N_q), int(d),
                                           int(block_n), int(bool(causal)))
    if rc < 0:
        _check(rc)
    return int(rc)


def fa_splitkv_workspace_bytes(B, H, N_q, d, num_splits):
    return int(load_library().fa_splitkv_workspace_bytes(B, H, N_q, d, num_splits))


def fa_splitkv_splits(B, H, N_q, N_k, d, causal):
    rc = load_library().fa_splitkv_splits(B, H, N_q, N_k, d, int(bool(causal)))
    if rc < 0:
        _check(rc)
    return rc


def fa_fwd_splitkv(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask, dtype,
                   num_splits, workspace, workspace_bytes, stream):
    """C fa_fwd_splitkv."""
    rc = load_library().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N_q,
                                       N_k, d, float(scale), int(bool(causal)), _ptr(kv_len_mask),
                                       int(dtype), int(num_splits), _ptr(workspace),
                                       int(workspace_bytes), stream)
    _check(rc)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, kv_len_mask,
                           dtype, num_splits, stream):
    """C fa_fwd_splitkv_noalloc: the split-key pass with its partial states in
    the library's own device scratch (no workspace, nothing allocated)."""
    rc = load_library().fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B,
                                               H, N_q, N_k, d, float(scale), int(bool(causal)),
                                               _ptr(kv_len_mask), int(dtype), int(num_splits),
                                               stream)
    _check(rc)


def fa_merge_states(m, l, acc, n_parts, rows, d, scale, o, lse, dtype, stream):
    """C fa_merge_states."""
    rc = load_library().fa_merge_states(_ptr(m), _ptr(l), _ptr(acc), int(n_parts), int(rows),
                                        int(d), float(scale), _ptr(o), _ptr(lse), int(dtype),
                                        stream)
    _check(rc)


def fa_softmax_rows(s, p, m, l, rows, n, dtype, stream):
    """C fa_softmax_rows."""
    rc = load_library().fa_softmax_rows(_ptr(s), _ptr(p), _ptr(m), _ptr(l), int(rows), int(n),
                                        int(dtype), stream)
    _check(rc)


def softmax_rows(s, out=None):
    """p, m, l for a float32 or bfloat16 CUDA tensor s whose last dimension is
    the row: p = softmax(s) along it (same shape and dtype), m the row maxima
    and l = sum exp(s - m) (float32, shape s.shape[:-1]).  out=s computes p
    in place."""
    import torch
    dt = _dtype_code(s)
    if not s.is_cuda or not s.is_contiguous() or s.dim() < 1:
        raise FaError(FA_ERR_SHAPE, "s must be a contiguous GPU tensor")
    n = s.shape[-1]
    rows = s.numel() // n if n else 0
    if out is None:
        p = torch.empty_like(s)
    else:
        _check_out("out", out, s.shape, s.dtype, s.device)
        p = out
    m = torch.empty(s.shape[:-1], dtype=torch.float32, device=s.device)
    l = torch.empty(s.shape[:-1], dtype=torch.float32, device=s.device)
    stream = torch.cuda.current_stream(s.device).cuda_stream
    fa_softmax_rows(s, p, m, l, rows, n, dt, stream)
    return p, m, l


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise FaError(FA_ERR_DTYPE, "tensors must be float32 or bfloat16")


def _check_qkv(q, k, v, kv_len_mask):
    import torch
    dt = _dtype_code(q)
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
    return dt, B, H, Nq, Nk, d


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output must be exactly what the kernels write: the C
    layer sees only a pointer, so a smaller or differently typed buffer would
    be written past its end."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise FaError(FA_ERR_SHAPE, "%s must be a torch tensor" % name)
    if t.dtype != dtype or t.device != device or not t.is_contiguous() or \
            tuple(t.shape) != tuple(shape):
        raise FaError(FA_ERR_SHAPE, "%s must be a contiguous %s tensor of shape %s on %s (got %s "
                      "%s%s on %s)" % (name, dtype, tuple(shape), device, t.dtype, tuple(t.shape),
                                       "" if t.is_contiguous() else ", not contiguous", t.device))


def _outputs(q, out):
    import torch
    B, H, Nq, _ = q.shape
    if out is not None:
        o, lse = out
        _check_out("o", o, q.shape, q.dtype, q.device)
        _check_out("lse", lse, (B, H, Nq), torch.float32, q.device)
        return o, lse
    return torch.empty_like(q), torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)


def attention_splitkv(q, k, v, scale=None, causal=False, kv_len_mask=None, num_splits=None,
                      out=None, workspace=None):
    """o, lse through fa_fwd_splitkv: the keys of every row cut into
    num_splits ranges (None: the library's choice, fa_splitkv_splits), whose
    partial states are merged.  The workspace (a uint8 CUDA tensor of at least
    fa_splitkv_workspace_bytes) is allocated with torch unless given."""
    import torch
    dt, B, H, Nq, Nk, d = _check_qkv(q, k, v, kv_len_mask)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if num_splits is None:
        num_splits = fa_splitkv_splits(B, H, Nq, Nk, d, causal)
    need = fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits)
    if need == 0:
        raise FaError(FA_ERR_ARG, "num_splits must be in 1..256")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.device != q.device
          or not workspace.is_contiguous()):
        raise FaError(FA_ERR_WORKSPACE, "workspace must be a contiguous tensor on %s" % q.device)
    o, lse = _outputs(q, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_len_mask, dt, num_splits,
                   workspace, workspace.numel() * workspace.element_size(), stream)
    return o, lse


def merge_states(m, l, acc, scale, out_dtype=None, out=None):
    """o, lse from partial states m, l [n_parts, rows] and acc
    [n_parts, rows, d] (contiguous float32 CUDA tensors, m in raw score units).
    o has dtype out_dtype (float32 or bfloat16; default float32)."""
    import torch
    n_parts, rows, d = acc.shape
    for name, t in (("m", m), ("l", l), ("acc", acc)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise FaError(FA_ERR_SHAPE, "%s must be a contiguous float32 GPU tensor" % name)
    if tuple(m.shape) != (n_parts, rows) or tuple(l.shape) != (n_parts, rows):
        raise FaError(FA_ERR_SHAPE, "m and l must be [n_parts, rows] matching acc")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        o = torch.empty(rows, d, dtype=out_dtype, device=acc.device)
        lse = torch.empty(rows, dtype=torch.float32, device=acc.device)
    else:
        o, lse = out
        _check_out("o", o, (rows, d), o.dtype, acc.device)
        _check_out("lse", lse, (rows,), torch.float32, acc.device)
    dt = _dtype_code(o)
    stream = torch.cuda.current_stream(acc.device).cuda_stream
    fa_merge_states(m, l, acc, n_parts, rows, d, scale, o, lse, dt, stream)
    return o, lse


def attention(q, k, v, scale=None, causal=False, kv_len_mask=None, block_n=0, reverse_kv=False,
              out=None, trace=None):
    """o, lse for torch tensors q [B,H,Nq,d], k, v [B,H,Nk,d] on one GPU.

    q, k, v: contiguous float32 or bfloat16 CUDA (HIP) tensors; kv_len_mask:
    None or a uint8 [B, Nk] CUDA tensor.  Outputs are allocated with torch
    (o in the input dtype, lse float32) unless `out=(o, lse)` is given.  The
    kernel runs on torch's current stream; nothing is synchronised.
    trace: None, or (buffer, b, h, row) with buffer a float32 CUDA tensor of
    ceil(N_k / block_n) * 4 elements: the per-tile state of that row
    (fa_opts.trace in include/fa.h).
    """
    import torch
    dt, B, H, Nq, Nk, d = _check_qkv(q, k, v, kv_len_mask)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    o, lse = _outputs(q, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = fa_opts(int(block_n), int(bool(reverse_kv)), None, 0, 0, 0)
    if trace is not None:
        buf, tb, th, trow = trace
        if buf.dtype != torch.float32 or not buf.is_cuda or not buf.is_contiguous():
            raise FaError(FA_ERR_SHAPE, "the trace buffer must be a contiguous float32 GPU tensor")
        bn = int(block_n) or 64
        if buf.numel() < (Nk + bn - 1) // bn * 4:
            raise FaError(FA_ERR_SHAPE, "the trace buffer needs ceil(N_k / block_n) * 4 floats")
        opts.trace, opts.trace_b, opts.trace_h, opts.trace_row = buf.data_ptr(), tb, th, trow
    fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_len_mask, dt, stream, opts)
    return o, lse
