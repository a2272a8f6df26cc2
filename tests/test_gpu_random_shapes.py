"""GPU parity over seeded random configurations: shapes with ragged tails,
both dtypes and head widths, causal or not, key-padding masks of every kind
(none, Bernoulli, per-batch prefix lengths, a visible span inside the range,
a fully masked batch), every tile size and order of the forward pass, the
split-key path with random split counts, and single query rows (the
decoding pass).  Every row is compared with the fp64 oracle."""

import os

import numpy as np
import pytest
import torch

import online_softmax_fa_amd as fa
from online_softmax_fa_amd import inputs
from _parity import compare, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# FA_RANDOM_CASES raises the count for a deeper sweep; configurations 0..119
# are the same at any count.
CASES = int(os.environ.get("FA_RANDOM_CASES", "120"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _config(i):
    """Configuration i, drawn from a generator seeded with i."""
    r = np.random.default_rng(7000 + i)
    single = r.random() < 0.2
    c = dict(
        B=int(r.integers(1, 4)), H=int(r.integers(1, 4)),
        Nk=int(r.integers(1, 700)), d=int(r.choice([64, 128])),
        dtype=str(r.choice(["f32", "bf16"])), causal=bool(r.random() < 0.4),
        mask=str(r.choice(["none", "bern", "prefix", "span", "dead"])),
        block_n=int(r.choice([0, 16, 32, 64, 128])), reverse=bool(r.random() < 0.3),
        splits=int(r.choice([0, 0, 2, 3, 7])),
    )
    c["Nq"] = 1 if single else (c["Nk"] if r.random() < 0.6 else int(r.integers(1, 700)))
    if single:
        c["dtype"], c["block_n"], c["reverse"] = "bf16", 0, False
    return c


def _mask(c, seed):
    B, Nk = c["B"], c["Nk"]
    kind = c["mask"]
    if kind == "none":
        return None
    if kind == "bern":
        return inputs.bernoulli_mask(B, Nk, 0.3, seed)
    if kind == "prefix":
        return inputs.prefix_mask(inputs.kv_lengths(B, Nk, seed, lo=1), Nk)
    m = torch.zeros(B, Nk, dtype=torch.uint8)
    if kind == "span":
        m[:, Nk // 4:max(Nk // 4 + 1, 3 * Nk // 4)] = 1
    else:                                  # dead: batch 0 sees nothing, the rest all keys
        m[1:] = 1
    return m


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(i):
    c = _config(i)
    seed = 7100 + i
    q, k, v = inputs.gaussian_qkv(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], seed, 1.0, c["dtype"])
    mask = _mask(c, seed + 1)
    scale = inputs.default_scale(c["d"])
    say("random %d: %s" % (i, c))
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=c["causal"], mask=mask)
    if c["splits"] and not c["reverse"] and c["block_n"] in (0, 64):
        md = None if mask is None else mask.to(DEV)
        o, lse = fa.attention_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale,
                                      causal=c["causal"], kv_len_mask=md, num_splits=c["splits"])
        torch.cuda.synchronize()
        o = o.float().cpu().numpy().astype(np.float64)
        lse = lse.cpu().numpy()
    else:
        o, lse = run_gpu(q, k, v, scale, causal=c["causal"], mask=mask, block_n=c["block_n"],
                         reverse_kv=c["reverse"])
    compare(o, lse, o_ref, lse_ref, c["dtype"], what="random %d" % i)
