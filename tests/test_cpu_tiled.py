"""The host-CPU tiled implementation (libfa_cpu.so) against the fp64 oracle.

These tests need no GPU.  The CPU kernel runs the pages' recurrence with the
exact running maximum over cache-sized tiles ("The math of FlashAttention",
"Why the same math matters on a CPU"); it must meet the same bars as the GPU
path: fp32 max |o - ref| <= 1e-5, bf16 max <= 2e-2 and mean <= 2e-3, lse
within 1e-3, fully masked rows exactly o = 0 and lse = -inf.
"""

import math
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
from online_softmax_fa_amd import cpu, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(cpu.LIB_PATH):
        pytest.fail("libfa_cpu.so is not built; run __graft_entry__.build()")
    oracle.build(force=False)


def _bits(t):
    """torch bf16 tensor -> uint16 numpy array of its bits."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(q, k, v, scale, causal=False, mask=None, dtype="f32", threads=0):
    if dtype == "bf16":
        o, lse, _ = cpu.attention_cpu(_bits(q), _bits(k), _bits(v), scale, causal, mask, threads,
                                      dtype="bf16")
        o = (o.astype(np.uint32) << 16).view(np.float32)
    else:
        o, lse, _ = cpu.attention_cpu(q.numpy(), k.numpy(), v.numpy(), scale, causal, mask, threads)
    ref_o, ref_lse, _ = oracle.attn_fwd(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                        scale, causal=causal, mask=mask)
    return o.astype(np.float64), lse, ref_o, ref_lse


def _compare(o, lse, ref_o, ref_lse, dtype, what=""):
    d = o.shape[-1]
    o, ref_o = o.reshape(-1, d), ref_o.reshape(-1, d)
    lse, ref_lse = lse.reshape(-1), ref_lse.reshape(-1)
    dead = np.isneginf(ref_lse)
    assert np.all(o[dead] == 0) and np.all(np.isneginf(lse[dead])), what
    live = ~dead
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[live])), what
    if live.any():
        err = np.abs(o[live] - ref_o[live])
        if dtype == "f32":
            assert err.max() <= 1e-5, (what, err.max())
        else:
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (what, err.max(), err.mean())
        assert np.abs(lse[live] - ref_lse[live]).max() <= 1e-3, what


def test_expf_accuracy():
    """The kernel's exp against the real exponential: within 2 ulp over the
    whole range that does not underflow, exp(0) = 1, exp(-inf) = 0."""
    xs = np.concatenate([-np.logspace(-9, np.log10(87.0), 3000),
                         np.linspace(-87.0, 0.0, 3001)]).astype(np.float32)
    worst = max(abs(cpu.cpu_expf(x) - math.exp(float(x))) / math.exp(float(x)) for x in xs)
    assert worst <= 2 * 2.0 ** -24, worst
    assert cpu.cpu_expf(0.0) == 1.0 and cpu.cpu_expf(float("-inf")) == 0.0
    assert cpu.cpu_expf(-200.0) == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small(dtype):
    w = inputs.workload("small", dtype=dtype)
    _compare(*_run(w["q"], w["k"], w["v"], w["scale"], dtype=dtype), dtype, "small")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adversarial_cases(dtype):
    """Exact scores: maximum in the last tile / first tile, a jump that
    underflows alpha, maxima straddling ln FLT_MAX; Bernoulli masks, the
    maximum's keys masked, causal with fully masked leading rows, all masked."""
    q, k, v = inputs.adversarial(dtype=dtype)
    for name, (mask, causal) in inputs.adversarial_cases().items():
        m = None if mask is None else mask.numpy()
        _compare(*_run(q, k, v, inputs.ADV_SCALE, causal, m, dtype), dtype, name)


@pytest.mark.parametrize("Nq,Nk,d", [(1, 1, 64), (1, 77, 128), (37, 5, 64), (130, 200, 96),
                                     (65, 65, 1), (33, 300, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes(Nq, Nk, d, causal):
    q, k, v = inputs.gaussian_qkv(2, 2, Nq, Nk, d, seed=4000 + Nq + Nk + d, dtype="f32")
    mask = inputs.bernoulli_mask(2, Nk, 0.3, seed=4100 + Nk).numpy()
    _compare(*_run(q, k, v, 1.0 / math.sqrt(d), causal, mask), "f32", "edge")


def test_threads_do_not_change_the_result():
    q, k, v = inputs.gaussian_qkv(1, 3, 200, 333, 64, seed=4200, dtype="f32")
    outs = [cpu.attention_cpu(q.numpy(), k.numpy(), v.numpy(), 0.125, True, None, t)
            for t in (1, 3, 8)]
    assert outs[0][2] == 1 and outs[1][2] == 3
    for o, lse, _ in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(lse, outs[0][1])


@pytest.mark.parametrize("isa", ["avx2", "base"])
def test_every_instruction_set_build(isa):
    """The AVX2 and baseline builds of the tile routine (the best build is
    the one the other tests run) on the adversarial and small cases, each in a
    fresh process because the choice is made once per process."""
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import test_cpu_tiled as t\n"
            "t.oracle.build(force=False)\n"
            "t.test_small('f32'); t.test_small('bf16')\n"
            "t.test_adversarial_cases('f32')\n"
            "t.test_edge_shapes(130, 200, 96, True)\n"
            "print('ok')\n") % (ROOT, os.path.join(ROOT, "tests"))
    env = dict(os.environ, FA_CPU_ISA=isa)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-3000:]


def test_argument_errors():
    lib = cpu.load_library()
    F = 0x10000
    args = lambda **kw: [kw.get("q", F), 2 * F, 3 * F, kw.get("o", 4 * F), 5 * F, kw.get("B", 1), 1,
                         8, 8, kw.get("d", 64), kw.get("scale", 0.1), 0, None, kw.get("dt", 0), 1]
    assert lib.fa_fwd_cpu(*args(q=None)) == -1
    assert lib.fa_fwd_cpu(*args(B=0)) == -2
    assert lib.fa_fwd_cpu(*args(d=300)) == -3
    assert lib.fa_fwd_cpu(*args(dt=2)) == -4
    assert lib.fa_fwd_cpu(*args(scale=-1.0)) == -5
    assert lib.fa_fwd_cpu(*args(o=F)) == -9


def test_exports_and_independence():
    """The library exports what include/fa_cpu.h declares, links neither the
    GPU runtime nor the oracle, and its source names neither."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa_cpu.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))
    assert declared == ["fa_cpu_expf", "fa_fwd_cpu"]
    out = subprocess.run(["nm", "-D", "--defined-only", cpu.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert set(declared) <= set(re.findall(r" T (fa_\w+)", out))
    deps = subprocess.run(["objdump", "-p", cpu.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "amdhip" not in deps and "faref" not in deps and "libfa.so" not in deps
    src = open(os.path.join(ROOT, "online_softmax_fa_amd", "csrc", "fa_cpu.cpp")).read()
    assert "oracle" not in src and "ref_attn" not in src
