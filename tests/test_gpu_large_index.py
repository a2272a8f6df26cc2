"""GPU parity where element offsets pass 2^31.

Two heads of N_k = 9 000 037 keys of width 128: K and V hold 2.3e9 elements
each (4.6 GB in bf16), so the key tiles at the end of head 1 lie past element
2^31, and one head's K alone (2.3e9 bytes) is too large for the decoding
pass's 32-bit offsets. A key-padding mask leaves the first and the last 500
keys of the sequence visible. The visible span is then the whole range, so
the kernels still walk every key tile in between. Masked keys contribute
nothing to the result (the oracle's own pins check that), so the oracle runs
on the 1000 visible keys alone, which keeps it to a second.
"""

import numpy as np
import pytest
import torch

import online_softmax_fa_amd as fa
from _parity import compare, run_oracle, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
H, NQ, NK, D = 2, 64, 9_000_037, 128
EDGE = 500
SCALE = 1.0 / D ** 0.5


@pytest.fixture(scope="module")
def case():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    say("large index space: B=1 H=%d N_q=%d N_k=%d d=%d bf16" % (H, NQ, NK, D))
    g = torch.Generator(device=DEV).manual_seed(9031)
    q = torch.randn(1, H, NQ, D, device=DEV, generator=g, dtype=torch.bfloat16)
    k = torch.randn(1, H, NK, D, device=DEV, generator=g, dtype=torch.bfloat16)
    v = torch.randn(1, H, NK, D, device=DEV, generator=g, dtype=torch.bfloat16)
    assert k.numel() > 2 ** 31 and NK * D * 2 >= 2 ** 31
    mask = torch.zeros(1, NK, dtype=torch.uint8, device=DEV)
    mask[:, :EDGE] = 1
    mask[:, NK - EDGE:] = 1
    keep = torch.cat([torch.arange(EDGE), torch.arange(NK - EDGE, NK)]).to(DEV)
    ks, vs = k[:, :, keep].cpu(), v[:, :, keep].cpu()
    o_ref, lse_ref = run_oracle(q.cpu(), ks, vs, SCALE)
    yield dict(q=q, k=k, v=v, mask=mask, o_ref=o_ref, lse_ref=lse_ref)
    del k, v
    torch.cuda.empty_cache()


def _np(o, lse):
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy()


def test_forward_past_2_31(case):
    o, lse = fa.attention(case["q"], case["k"], case["v"], scale=SCALE, kv_len_mask=case["mask"])
    o, lse = _np(o, lse)
    compare(o, lse, case["o_ref"], case["lse_ref"], "bf16", what="forward")


def test_splitkv_past_2_31(case):
    o, lse = fa.attention_splitkv(case["q"], case["k"], case["v"], scale=SCALE,
                                  kv_len_mask=case["mask"], num_splits=8)
    o, lse = _np(o, lse)
    compare(o, lse, case["o_ref"], case["lse_ref"], "bf16", what="split-key, 8 ranges")


def test_single_row_past_2_31(case):
    # one query row: too large for the decoding pass, so the forward kernel runs
    q1 = case["q"][:, :, :1].contiguous()
    for name, call in (("forward", fa.attention), ("split-key", fa.attention_splitkv)):
        o, lse = call(q1, case["k"], case["v"], scale=SCALE, kv_len_mask=case["mask"])
        o, lse = _np(o, lse)
        compare(o, lse, case["o_ref"][:, :, :1], case["lse_ref"][:, :, :1], "bf16",
                what="one row, " + name)
