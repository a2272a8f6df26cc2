"""fa_fwd_splitkv_noalloc, the split-key pass for callers that cannot
allocate: its partial states live in the library's own device scratch instead
of a caller-supplied workspace.  Called through the C ABI, it must give what
fa_fwd_splitkv gives with a workspace on the same inputs and split count
(the same kernels, so bit for bit), and both must meet the oracle's bars.
Two calls in a row, the second smaller, show that what the first left in the
scratch does not leak into the second."""

import ctypes

import numpy as np
import pytest
import torch

import online_softmax_fa_amd as fa
from online_softmax_fa_amd import inputs
from _parity import compare, run_oracle, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SCRATCH_BYTES = 32 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _call_both(q, k, v, scale, causal, mask, splits, dtype):
    """The no-alloc entry point and fa_fwd_splitkv with a torch workspace,
    each through the C ABI on torch's current stream."""
    qd, kd, vd = (x.contiguous().to(DEV) for x in (q, k, v))
    md = None if mask is None else mask.contiguous().to(DEV)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32
    stream = torch.cuda.current_stream(DEV).cuda_stream
    lib = fa.load_library()
    o1 = torch.full_like(qd, float("nan"))
    lse1 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    rc = lib.fa_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                                    lse1.data_ptr(), B, H, Nq, Nk, d, ctypes.c_float(scale),
                                    int(causal), None if md is None else md.data_ptr(), dt,
                                    splits, ctypes.c_void_p(stream))
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    need = fa.fa_splitkv_workspace_bytes(B, H, Nq, d, splits)
    assert 0 < need <= SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o2 = torch.full_like(qd, float("nan"))
    lse2 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    rc = lib.fa_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
                            lse2.data_ptr(), B, H, Nq, Nk, d, ctypes.c_float(scale), int(causal),
                            None if md is None else md.data_ptr(), dt, splits, ws.data_ptr(),
                            need, ctypes.c_void_p(stream))
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    return o1, lse1, o2, lse2


def _check_case(q, k, v, scale, causal, mask, splits, dtype, what):
    say("no-alloc %s: B,H,Nq,Nk,d=%s splits=%d" % (what, (q.shape[0], q.shape[1], q.shape[2],
                                                         k.shape[2], q.shape[3]), splits))
    o1, lse1, o2, lse2 = _call_both(q, k, v, scale, causal, mask, splits, dtype)
    # same kernels and split count: identical bits
    assert torch.equal(o1.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o2.view(torch.int16 if dtype == "bf16" else torch.int32)), what
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32)), what
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask)
    compare(o1.float().cpu().numpy().astype(np.float64), lse1.cpu().numpy(), o_ref, lse_ref,
            dtype, what=what)


def test_noalloc_matches_workspace_path_twice():
    """A decode-shaped call (one query row, bf16, the decoding pass) with
    per-batch key lengths and a fully masked batch, then a smaller
    prefill-shaped causal call through the forward kernel in split mode,
    fp32, with a different split count."""
    B, H, Nq, Nk, d = 4, 8, 1, 4099, 128
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=7100, dtype="bf16")
    lens = inputs.kv_lengths(B, Nk, seed=7101, lo=1)
    mask = inputs.prefix_mask(lens, Nk)
    mask[3] = 0
    _check_case(q, k, v, inputs.default_scale(d), False, mask, 16, "bf16", "decode")

    q, k, v = inputs.gaussian_qkv(1, 2, 300, 300, 64, seed=7102, dtype="f32")
    _check_case(q, k, v, inputs.default_scale(64), True, None, 3, "f32", "prefill")


def test_noalloc_rejects_requests_beyond_the_scratch():
    """Partial states larger than the scratch give FA_ERR_SCRATCH before
    anything is enqueued: the outputs stay as they were."""
    B, H, Nq, Nk, d, splits = 2, 16, 1024, 1024, 128, 16
    assert fa.fa_splitkv_workspace_bytes(B, H, Nq, d, splits) > SCRATCH_BYTES
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=7103, dtype="bf16")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.zeros_like(qd)
    lse = torch.zeros(B, H, Nq, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_noalloc(qd, kd, vd, o, lse, B, H, Nq, Nk, d, inputs.default_scale(d),
                                  False, None, fa.FA_DTYPE_BF16, splits,
                                  torch.cuda.current_stream(DEV).cuda_stream)
    assert e.value.code == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0 and int(torch.count_nonzero(lse)) == 0
