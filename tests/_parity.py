"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same inputs, compare at the stated bars.

Bars (O upcast to fp64; lse in fp32 against the fp64 oracle):
  fp32 inputs: max |o - o_ref| <= 1e-5
  bf16 inputs: max |o - o_ref| <= 2e-2 and mean |o - o_ref| <= 2e-3
  both:        max |lse - lse_ref| <= 1e-3
  rows with no visible key: o exactly 0 and lse exactly -inf
  no NaN or Inf anywhere else
"""

import sys

import numpy as np
import torch

import oracle
import online_softmax_fa_amd as fa

TOL = {"f32": dict(max_abs=1e-5, mean_abs=None), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}


def header_define(name):
    """The integer value of a #define in include/fa.h (the bounds the library
    documents are read from the header, not restated)."""
    import os
    import re
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                        "fa.h")
    m = re.search(r"^#define\s+%s\s+(\d+)\s*$" % name, open(path).read(), re.M)
    assert m, name
    return int(m.group(1))
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def to_np32(t):
    return t.detach().to("cpu").float().numpy()


def run_gpu(q, k, v, scale, causal=False, mask=None, block_n=0, reverse_kv=False):
    """Inputs are CPU tensors; returns (o as fp64 numpy, lse as fp32 numpy)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.contiguous().to(dev) for x in (q, k, v))
    md = None if mask is None else mask.contiguous().to(dev)
    o, lse = fa.attention(qd, kd, vd, scale=scale, causal=causal, kv_len_mask=md,
                          block_n=block_n, reverse_kv=reverse_kv)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy()


def run_oracle(q, k, v, scale, causal=False, mask=None, rows=None):
    m = None if mask is None else mask.numpy()
    o, lse, _ = oracle.attn_fwd(to_np32(q), to_np32(k), to_np32(v), scale, causal=causal, mask=m,
                                rows=rows)
    return o, lse


def compare(o, lse, o_ref, lse_ref, dt, max_abs=None, mean_abs=None, lse_tol=LSE_TOL, what=""):
    """o/lse and o_ref/lse_ref: matching shapes ([..., d] and [...])."""
    max_abs = TOL[dt]["max_abs"] if max_abs is None else max_abs
    mean_abs = TOL[dt]["mean_abs"] if mean_abs is None else mean_abs
    o = o.reshape(-1, o.shape[-1])
    o_ref = o_ref.reshape(-1, o_ref.shape[-1])
    lse = lse.reshape(-1).astype(np.float64)
    lse_ref = lse_ref.reshape(-1)
    dead = np.isneginf(lse_ref)
    live = ~dead
    assert np.all(o[dead] == 0.0), "%s: fully masked rows must give o = 0" % what
    assert np.all(np.isneginf(lse[dead])), "%s: fully masked rows must give lse = -inf" % what
    assert np.all(np.isfinite(o)), "%s: NaN/Inf in o" % what
    assert np.all(np.isfinite(lse[live])), "%s: NaN/Inf in lse of a live row" % what
    stats = {}
    if live.any():
        err = np.abs(o[live] - o_ref[live])
        stats["max_abs"] = float(err.max())
        stats["mean_abs"] = float(err.mean())
        stats["lse_max_abs"] = float(np.abs(lse[live] - lse_ref[live]).max())
        assert stats["max_abs"] <= max_abs, "%s: max |o - ref| = %.3e > %.1e" % (
            what, stats["max_abs"], max_abs)
        if mean_abs is not None:
            assert stats["mean_abs"] <= mean_abs, "%s: mean |o - ref| = %.3e > %.1e" % (
                what, stats["mean_abs"], mean_abs)
        assert stats["lse_max_abs"] <= lse_tol, "%s: max |lse - ref| = %.3e > %.1e" % (
            what, stats["lse_max_abs"], lse_tol)
    say("  %s: %s" % (what, ", ".join("%s=%.3e" % kv for kv in stats.items())))
    log_margins(what, dt, stats, max_abs, mean_abs, lse_tol, int(live.sum()), int(dead.sum()))
    return stats


def log_margins(what, dt, stats, max_abs, mean_abs, lse_tol, rows, dead_rows):
    """With FA_PARITY_LOG set, append one JSON line per comparison (the test,
    the case, the achieved errors and the bars) to that file: the source of
    the committed per-configuration margin summary."""
    import json
    import os
    path = os.environ.get("FA_PARITY_LOG")
    if not path:
        return
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").rsplit(" ", 1)[0], "case": what,
           "dtype": dt, "rows": rows, "rows_without_visible_key": dead_rows,
           "bars": {"max_abs": max_abs, "mean_abs": mean_abs, "lse_max_abs": lse_tol}}
    rec.update(stats)
    with open(path, "a") as fh:
        fh.write(json.dumps(rec) + "\n")


def sample_rows(B, H, N, heads, n_random, seed):
    """Flat row indices: for each (b, h) in `heads`, the first and last 128 rows
    plus n_random random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    for (b, h) in heads:
        base = (b * H + h) * N
        idx = set(range(min(128, N))) | set(range(max(0, N - 128), N))
        idx |= set(rng.integers(0, N, n_random).tolist())
        rows.extend(base + i for i in sorted(idx))
    return np.array(rows, dtype=np.int64)
