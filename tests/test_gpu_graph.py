"""The library's calls captured in a HIP graph (torch.cuda.graph) and
replayed.  The entry points allocate nothing, clear nothing and never
synchronise, so a captured launch is the same kernel on the same buffers.
Each graph is replayed several times with new inputs copied into the
captured buffers between replays (eager work and a synchronisation in
between); every replay must equal an eager call on the same inputs bit for
bit, and the eager call must itself match the oracle."""

import numpy as np
import pytest
import torch

import online_softmax_fa_amd as fa
import oracle
from online_softmax_fa_amd import inputs
from _parity import compare, run_oracle, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _replay_and_check(fill, capture, eager, outputs):
    """fill(r): writes input set r into the captured buffers; capture(): the
    calls to record; eager(): the same calls into fresh outputs; outputs():
    the captured outputs."""
    fill(0)
    capture()                      # first call outside the graph (kernel set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        fill(r + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs()]
        want = eager()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), "replay %d differs from the eager call" % r
    return g


@pytest.mark.parametrize("causal", [False, True])
def test_graph_fwd(causal):
    B, H, N, d = 2, 4, 640, 128
    sets = [inputs.gaussian_qkv(B, H, N, N, d, 6100 + r, 1.0, "bf16") for r in range(REPLAYS + 1)]
    mask = inputs.bernoulli_mask(B, N, 0.2, 6199).to(DEV)
    scale = inputs.default_scale(d)
    q, k, v = (torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)

    def fill(r):
        for dst, src in zip((q, k, v), sets[r]):
            dst.copy_(src)

    def capture():
        fa.attention(q, k, v, scale=scale, causal=causal, kv_len_mask=mask, out=(o, lse))

    def eager():
        return fa.attention(q, k, v, scale=scale, causal=causal, kv_len_mask=mask)

    say("graph fwd causal=%d" % causal)
    _replay_and_check(fill, capture, eager, lambda: (o, lse))
    qs, ks, vs = sets[REPLAYS]
    o_ref, lse_ref = run_oracle(qs, ks, vs, scale, causal=causal, mask=mask.cpu())
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
            what="graph fwd")


def test_graph_splitkv():
    B, H, Nq, Nk, d, ns = 2, 4, 3, 4099, 128, 7
    sets = [inputs.gaussian_qkv(B, H, Nq, Nk, d, 6200 + r, 0.5, "bf16") for r in range(REPLAYS + 1)]
    scale = inputs.default_scale(d)
    q = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=DEV)
    k, v = (torch.empty(B, H, Nk, d, dtype=torch.bfloat16, device=DEV) for _ in range(2))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(B, H, Nq, d, ns), dtype=torch.uint8, device=DEV)

    def fill(r):
        for dst, src in zip((q, k, v), sets[r]):
            dst.copy_(src)

    def capture():
        fa.attention_splitkv(q, k, v, scale=scale, num_splits=ns, out=(o, lse), workspace=ws)

    def eager():
        return fa.attention_splitkv(q, k, v, scale=scale, num_splits=ns)

    say("graph split-key splits=%d" % ns)
    _replay_and_check(fill, capture, eager, lambda: (o, lse))
    qs, ks, vs = sets[REPLAYS]
    o_ref, lse_ref = run_oracle(qs, ks, vs, scale)
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
            what="graph split")


def test_graph_softmax_rows():
    rows, n = 300, 1000
    sets = [inputs.gaussian((rows, n), 6300 + r, 3.0) for r in range(REPLAYS + 1)]
    s = torch.empty(rows, n, dtype=torch.float32, device=DEV)
    p = torch.empty_like(s)
    bufs = {}

    def fill(r):
        s.copy_(sets[r])

    def capture():
        bufs["out"] = fa.softmax_rows(s, out=p)

    def eager():
        return fa.softmax_rows(s)

    say("graph softmax rows")
    _replay_and_check(fill, capture, eager, lambda: bufs["out"])
    got = p.cpu().numpy()
    for r in (0, 151, rows - 1):
        ref, _, _ = oracle.softmax_row(sets[REPLAYS][r].numpy().astype(np.float64))
        assert np.max(np.abs(got[r] - ref)) <= 1e-6


def test_calls_run_on_the_callers_stream():
    """Every entry point enqueues on the stream it is given (torch's current
    stream for the binding): work on a side stream, ordered after the inputs
    are written there and before the outputs are read there, gives the same
    bits as on the default stream."""
    B, H, N, d = 1, 2, 777, 128
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, 6400, 1.0, "bf16")
    scale = inputs.default_scale(d)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o0, l0 = fa.attention(qd, kd, vd, scale=scale, causal=True)
    s0, _ = fa.attention_splitkv(qd[:, :, :1].contiguous(), kd, vd, scale=scale, num_splits=5)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        q2, k2, v2 = (x.to(DEV, non_blocking=False) for x in (q, k, v))
        o1, l1 = fa.attention(q2, k2, v2, scale=scale, causal=True)
        s1, _ = fa.attention_splitkv(q2[:, :, :1].contiguous(), k2, v2, scale=scale, num_splits=5)
        got = (o1.clone(), l1.clone(), s1.clone())
    side.synchronize()
    assert torch.equal(got[0], o0) and torch.equal(got[1], l0) and torch.equal(got[2], s0)
