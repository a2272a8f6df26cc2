"""GPU per-tile trace of one row (fa_opts.trace) against the oracle's
block-by-block recurrence.

The tiled-attention interview answer recommends printing (m, l) after every
block when debugging; the kernel writes {tile, m, l, 0} for one chosen row
after each key tile it visits.  With exact scores (the adversarial heads) the
fp32 kernel's m must equal the oracle's running maximum and its l the oracle's
l ("2.2b", "The Complete Online Softmax Algorithm"), for every tile size, both
traversal orders and the causal diagonal.  The bf16 kernel states l against a
reference that may lag the maximum, so it is compared through the running log
of the sum of exponentials, m*scale + ln l, which any reference gives alike,
and its reference is checked against the documented lag bound.
"""

import math

import numpy as np
import pytest
import torch

from oracle.online import online_attention_row
from online_softmax_fa_amd import inputs
import online_softmax_fa_amd as fa
from _parity import header_define, say, to_np32

LAG_LOG2 = header_define("FA_BF16_REF_LAG_LOG2")

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _tiles_visited(row, N, bn, causal, bm, mask_row=None):
    """Key tiles the row's workgroup visits, as (first, count): all of them,
    or under causality those up to the diagonal of the last row of its query
    tile of bm rows; with a key-padding mask only those from the first to the
    last visible key of that range (none if it has no visible key)."""
    n = (N + bn - 1) // bn
    if causal:
        q0 = row // bm * bm
        n = min(n, (min(q0 + bm, N) - 1) // bn + 1)
    if mask_row is None:
        return 0, n
    vis = np.flatnonzero(np.asarray(mask_row)[: min(N, n * bn)])
    if len(vis) == 0:
        return 0, 0
    return vis[0] // bn, vis[-1] // bn + 1 - vis[0] // bn


def _trace(qd, kd, vd, scale, causal, mask, bn, rev, b, h, row):
    N = kd.shape[2]
    buf = torch.full(((N + bn - 1) // bn * 4,), float("nan"), device=DEV)
    o, lse = fa.attention(qd, kd, vd, scale=scale, causal=causal, kv_len_mask=mask, block_n=bn,
                          reverse_kv=rev, trace=(buf, b, h, row))
    torch.cuda.synchronize()
    return buf.cpu().numpy().reshape(-1, 4), o, lse


def _oracle_trace(s_row, vis, bn, t0, n_t, rev):
    """The oracle's recurrence over key tiles t0 .. t0 + n_t - 1 (the keys
    before and after them are masked), block indices renumbered to tiles."""
    lo, hi = t0 * bn, min(len(s_row), (t0 + n_t) * bn)
    order = list(range(n_t))
    if rev:
        order = order[::-1]
    ref = online_attention_row(s_row[lo:hi], None, block=bn, order=order, visible=vis[lo:hi])
    for e in ref["trace"]:
        e["block"] += t0
    return ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bn", [16, 32, 64, 128])
@pytest.mark.parametrize("rev", [False, True])
def test_trace_of_adversarial_rows(dtype, bn, rev):
    q, k, v = inputs.adversarial(dtype=dtype)
    scale = inputs.ADV_SCALE
    c = scale * LOG2E
    qn, kn = to_np32(q).astype(np.float64)[0], to_np32(k).astype(np.float64)[0]
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    N = k.shape[2]
    cases = inputs.adversarial_cases()
    for name in ("nomask", "causal", "bern30", "mask_max_keys", "causal_prefix_masked",
                 "all_masked"):
        mask, causal = cases[name]
        md = None if mask is None else mask.to(DEV)
        for h in (0, 2, 3):
            for row in (0, 37, 500, N - 1):
                say("trace %s bn=%d rev=%d %s head %d row %d" % (dtype, bn, rev, name, h, row))
                tr, _, _ = _trace(qd, kd, vd, scale, causal, md, bn, rev, 0, h, row)
                bm = fa.fa_query_tile_rows(fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32,
                                           q.shape[0], q.shape[1], q.shape[2], q.shape[3], bn,
                                           causal)
                t0, n_t = _tiles_visited(row, N, bn, causal, bm,
                                         None if mask is None else mask[0].numpy())
                assert np.all(np.isfinite(tr[:n_t, 0])) and np.all(np.isnan(tr[n_t:]))
                s_row = scale * (kn[h] @ qn[h, row])
                vis = np.ones(N, bool) if mask is None else mask[0].numpy().astype(bool)
                if causal:
                    vis &= np.arange(N) <= row
                ref = _oracle_trace(s_row, vis, bn, t0, n_t, rev)["trace"]
                assert [int(t) for t in tr[:n_t, 0]] == [e["block"] for e in ref]
                for e, (t, m, l, _) in zip(ref, tr[:n_t]):
                    if e["m_new"] == -math.inf:
                        assert m == -math.inf and l == 0.0
                        continue
                    lse_k = m * scale + math.log(l)
                    lse_o = e["m_new"] + math.log(e["l"])
                    if dtype == "f32":
                        assert m * scale == e["m_new"]            # exact scores, exact max
                        assert abs(l - e["l"]) <= 1e-5 * e["l"]
                    else:
                        m_true = e["m_new"] / scale
                        slack = 1e-6 * abs(m_true) + 1e-6         # rounding of mc / c
                        assert m <= m_true + slack
                        # lag bound of the header: the fast path keeps weights
                        # up to 2^FA_BF16_REF_LAG_LOG2
                        assert m >= m_true - LAG_LOG2 / c - slack
                    assert abs(lse_k - lse_o) <= 1e-5 * max(1.0, abs(lse_o))


def test_trace_of_gaussian_causal_rows():
    """bf16 random inputs at the production tile size: the running log-sum
    of every visited tile within the lse bar."""
    B, H, N, d = 1, 2, 2048, 64
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, seed=2900, dtype="bf16")
    scale = inputs.default_scale(d)
    qn, kn = to_np32(q).astype(np.float64)[0], to_np32(k).astype(np.float64)[0]
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    for h, row in ((0, 0), (0, 129), (1, 1000), (1, 2047)):
        tr, _, _ = _trace(qd, kd, vd, scale, True, None, 64, False, 0, h, row)
        t0, n_t = _tiles_visited(row, N, 64, True,
                                 fa.fa_query_tile_rows(fa.FA_DTYPE_BF16, B, H, N, d, 64, True))
        s_row = scale * (kn[h] @ qn[h, row])
        vis = np.arange(N) <= row
        ref = _oracle_trace(s_row, vis, 64, t0, n_t, False)["trace"]
        for e, (t, m, l, _) in zip(ref, tr[:n_t]):
            if e["m_new"] == -math.inf:
                assert m == -math.inf and l == 0.0
            else:
                assert abs(m * scale + math.log(l) - (e["m_new"] + math.log(e["l"]))) <= 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trace_leaves_the_result_unchanged(dtype):
    q, k, v = inputs.gaussian_qkv(2, 3, 300, 300, 128, seed=2950, dtype=dtype)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    scale = inputs.default_scale(128)
    o0, lse0 = fa.attention(qd, kd, vd, scale=scale, causal=True)
    _, o1, lse1 = _trace(qd, kd, vd, scale, True, None, 64, False, 1, 2, 150)
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)


def test_trace_in_paired_workgroups():
    """Causal bf16 launch whose 256-row query tiles go in pairs (t, n-1-t), one
    workgroup taking both in turn (B=4 H=256 N=257 d=128: 1024 pairs on 256
    CUs): the trace of a row in the first item of a pair (tile 1) and in the
    second (tile 0) follows the oracle's recurrence, and tracing leaves the
    result unchanged."""
    B, H, N, d = 4, 256, 257, 128
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, seed=2990, dtype="bf16")
    scale = inputs.default_scale(d)
    c = scale * LOG2E
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    bm = fa.fa_query_tile_rows(fa.FA_DTYPE_BF16, B, H, N, d, 64, True)
    o0, lse0 = fa.attention(qd, kd, vd, scale=scale, causal=True)
    for b, h, row in ((0, 0, 0), (1, 7, 200), (2, 100, 256), (3, 255, 255)):
        say("paired trace b %d h %d row %d" % (b, h, row))
        tr, o1, lse1 = _trace(qd, kd, vd, scale, True, None, 64, False, b, h, row)
        assert torch.equal(o0, o1) and torch.equal(lse0, lse1)
        t0, n_t = _tiles_visited(row, N, 64, True, bm)
        assert np.all(np.isfinite(tr[:n_t, 0])) and np.all(np.isnan(tr[n_t:]))
        qn = to_np32(q[b, h]).astype(np.float64)
        kn = to_np32(k[b, h]).astype(np.float64)
        s_row = scale * (kn @ qn[row])
        vis = np.arange(N) <= row
        ref = _oracle_trace(s_row, vis, 64, t0, n_t, False)["trace"]
        assert [int(t) for t in tr[:n_t, 0]] == [e["block"] for e in ref]
        for e, (t, m, l, _) in zip(ref, tr[:n_t]):
            if e["m_new"] == -math.inf:
                assert m == -math.inf and l == 0.0
                continue
            m_true = e["m_new"] / scale
            slack = 1e-6 * abs(m_true) + 1e-6
            assert m_true - LAG_LOG2 / c - slack <= m <= m_true + slack
            assert abs(m * scale + math.log(l) - (e["m_new"] + math.log(e["l"]))) <= 1e-3
