"""GPU parity of fa_softmax_rows, the online softmax over score rows.

The kernel runs the pages' recurrence with the values removed: one pass for
the running (m, l), one that writes p = exp(s - m) / l ("2.2b: FlashAttention
-- Online Softmax", "The Challenge: Computing m and l in Blocks" through "When
Rescaling Actually Happens").  The oracle is the fp64 three-pass safe softmax
of each row (oracle.softmax_row).  Rows cover the pages' toy row, every path of
the kernel (rows held in registers between the passes, longer rows read
twice, unaligned rows, short rows), masked
(-inf) entries, fully masked rows, scores far beyond exp's range, and
in-place use.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import online_softmax_fa_amd as fa
from online_softmax_fa_amd import inputs
from _parity import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))
BAR = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _check(s_cpu, p, m, l, dt, what):
    """s_cpu: [rows, n] float32 (the exact values the GPU saw)."""
    s64 = s_cpu.numpy().astype(np.float64)
    p = p.float().cpu().numpy().astype(np.float64)
    m, l = m.cpu().numpy(), l.cpu().numpy()
    max_bar, mean_bar = BAR[dt]
    errs = []
    for r in range(s64.shape[0]):
        vis = np.isfinite(s64[r])
        p_ref, m_ref, l_ref = oracle.softmax_row(np.where(vis, s64[r], 0.0), vis)
        if not vis.any():
            assert np.all(p[r] == 0) and m[r] == -np.inf and l[r] == 0.0, what
            continue
        assert m[r] == m_ref, what                       # the maximum of the inputs, exactly
        assert abs(l[r] - l_ref) <= 1e-5 * l_ref, what
        assert np.all(p[r][~vis] == 0.0), what
        errs.append(np.abs(p[r] - p_ref))
    if errs:
        e = np.concatenate(errs)
        say("  %s: max %.2e mean %.2e" % (what, e.max(), e.mean()))
        assert e.max() <= max_bar, what
        if mean_bar is not None:
            assert e.mean() <= mean_bar, what


def _run(s_cpu, dt, out_inplace=False):
    t = s_cpu.to(inputs.TORCH_DTYPE[dt]).to(DEV)
    seen = t.float().cpu()                            # what the kernel sees (bf16-rounded)
    if out_inplace:
        p, m, l = fa.softmax_rows(t, out=t)
    else:
        p, m, l = fa.softmax_rows(t)
    torch.cuda.synchronize()
    return seen, p, m, l


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_pages_toy_row(dt):
    """S = [2, 4, 1, 3] -> [0.087, 0.644, 0.032, 0.237] ("2.2b", "The Softmax
    Formula"), at half a unit of the printed digit, and against the oracle."""
    c = [x for x in GOLDEN["softmax_rows"] if x["id"] == "toy1_softmax"][0]
    s = torch.tensor([c["scores"]], dtype=torch.float32)
    seen, p, m, l = _run(s, dt)
    tol = c["p_tol"] + (0.0 if dt == "f32" else 2.0 ** -9)
    assert np.max(np.abs(p.float().cpu().numpy()[0] - np.array(c["p"]))) <= tol
    assert float(m[0]) == c["m"]
    assert abs(float(l[0]) - c["l"]) <= c["l_tol"]
    _check(seen, p, m, l, dt, "toy")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,n", [(1, 1), (3, 5), (7, 1000), (64, 1001), (33, 8192),
                                    (5, 100003), (300, 64), (4, 40000)])
@pytest.mark.parametrize("sigma", [1.0, 30.0])
def test_random_rows(dt, rows, n, sigma):
    g = torch.Generator().manual_seed(3000 + rows + n)
    s = torch.randn(rows, n, generator=g) * sigma
    masked = torch.rand(rows, n, generator=g) < 0.3
    s[masked] = -float("inf")
    if rows > 2:
        s[1] = -float("inf")                          # a fully masked row
        s[2] += 1.0e4                                 # far beyond exp's range
        s[0, 0] = 500.0                               # a lone huge entry
    seen, p, m, l = _run(s, dt)
    _check(seen, p, m, l, dt, "%s %dx%d sigma %g" % (dt, rows, n, sigma))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_in_place_matches_out_of_place(dt):
    g = torch.Generator().manual_seed(3100)
    s = torch.randn(17, 4096, generator=g) * 5
    _, p0, m0, l0 = _run(s, dt)
    _, p1, m1, l1 = _run(s, dt, out_inplace=True)
    assert torch.equal(p0, p1) and torch.equal(m0, m1) and torch.equal(l0, l1)


def test_unaligned_rows():
    """A row start that is not 16-byte aligned takes the element-wise path."""
    g = torch.Generator().manual_seed(3200)
    base = (torch.randn(4 * 513 + 1, generator=g) * 3).to(DEV)
    s = base[1:].view(4, 513)                         # 4-byte offset from the allocation
    assert s.data_ptr() % 16 != 0
    p, m, l = fa.softmax_rows(s)
    torch.cuda.synchronize()
    _check(s.cpu(), p, m, l, "f32", "unaligned")
