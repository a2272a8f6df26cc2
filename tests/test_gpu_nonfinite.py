"""Keys hidden by the key-padding mask contribute exactly zero whatever their
k and v rows hold: padded cache slots may contain NaN, +Inf, -Inf or any other
bits ("The math of FlashAttention", "Pitfalls in implementing the
recurrence": masks go in before the maximum; tiled-attention interview answer,
second paragraph: masked keys contribute zero).  A masked key's weight is 0,
and 0 times a non-finite value would be NaN, so the kernels must never form
that product.  The oracle skips hidden keys, so its result is the plain one
over the visible keys; every path is compared with it at the usual bars:
the forward kernels at every tile size and both orders, the split-key pass,
the decoding pass (one query row) and the merge."""

import numpy as np
import pytest
import torch

import online_softmax_fa_amd as fa
from online_softmax_fa_amd import inputs
from _parity import compare, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
POISON = (float("nan"), float("inf"), float("-inf"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _poisoned(B, H, Nq, Nk, d, dtype, seed):
    """Gaussian q, k, v and a key-padding mask (batch 0: a prefix of 60% of
    the keys; batch 1: 35% of the keys masked at random, the last key among
    them); the k and v rows of every masked key cycle through NaN, +Inf and
    -Inf, element by element."""
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=seed, dtype=dtype)
    mask = inputs.bernoulli_mask(B, Nk, 0.35, seed + 1)
    mask[0] = inputs.prefix_mask(torch.tensor([int(0.6 * Nk)]), Nk)[0]
    mask[1, Nk - 1] = 0
    hidden = (mask == 0).nonzero().tolist()
    fill = torch.tensor([POISON[i % 3] for i in range(d)], dtype=k.dtype)
    for n, (b, j) in enumerate(hidden):
        k[b, :, j, :] = torch.roll(fill, n)
        v[b, :, j, :] = torch.roll(fill, n + 1)
    assert not torch.isfinite(k.float()).all() and not torch.isfinite(v.float()).all()
    return q, k, v, mask


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_with_nonfinite_masked_keys(dtype, causal, d):
    B, H, N = 2, 2, 333
    q, k, v, mask = _poisoned(B, H, N, N, d, dtype, seed=8200 + d + causal)
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask)
    for bn in (0, 16, 32, 64, 128):
        for rev in (False, True):
            say("non-finite masked keys %s causal=%d d=%d bn=%d rev=%d" % (dtype, causal, d, bn,
                                                                          rev))
            o, lse = run_gpu(q, k, v, scale, causal=causal, mask=mask, block_n=bn, reverse_kv=rev)
            compare(o, lse, o_ref, lse_ref, dtype, what="bn%d rev%d" % (bn, rev))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_forward_with_nonfinite_masked_keys(dtype):
    """A shape that takes the 8-wave, 256-row workgroups of the bf16 kernel."""
    B, H, N, d = 2, 64, 1000, 128
    q, k, v, mask = _poisoned(B, H, N, N, d, dtype, seed=8300)
    scale = inputs.default_scale(d)
    rows = np.concatenate([np.arange(0, 300), (B * H - 1) * N + np.arange(N - 300, N)])
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=True, mask=mask, rows=rows)
    o, lse = run_gpu(q, k, v, scale, causal=True, mask=mask)
    compare(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype, what="8-wave")


@pytest.mark.parametrize("Nq", [1, 40])
def test_splitkv_and_decode_with_nonfinite_masked_keys(Nq):
    """The split-key pass (and, for one query row, the decoding pass that
    streams K and V through registers) with its merge."""
    B, H, Nk, d = 2, 3, 4099, 128
    q, k, v, mask = _poisoned(B, H, Nq, Nk, d, "bf16", seed=8400 + Nq)
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, mask=mask)
    qd, kd, vd, md = (x.to(DEV) for x in (q, k, v, mask))
    for splits in (None, 1, 5):
        say("split/decode non-finite Nq=%d splits=%s" % (Nq, splits))
        o, lse = fa.attention_splitkv(qd, kd, vd, scale=scale, kv_len_mask=md, num_splits=splits)
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), o_ref, lse_ref,
                "bf16", what="splits %s" % splits)
    o, lse = run_gpu(q, k, v, scale, mask=mask)
    compare(o, lse, o_ref, lse_ref, "bf16", what="fa_fwd")
