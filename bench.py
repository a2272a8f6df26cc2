"""Throughput of the exact attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (every query row of every
head), with Q, K, V already resident in HBM.  The default workload is the
headline one: B=2, H=32, N_q=N_k=8192, d=128, bf16, causal.

The defaults (200 timed launches after 50 warm-up ones, about a quarter of a
second of GPU time) let the clocks settle: twenty launches after five read
about 7% slower on the same device.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      attention TFLOP/s = 4*B*H*N_q*N_k*d / t, halved for causal
  roofline   the kernel against the bf16 dense MFMA peak (2.5 PFLOP/s)
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload's rows, on this host's cores, in the same unit

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--block-n BN] [--no-cpu-baseline] [--cpu-seconds S]
       python bench.py --copy-calibration MIB
           runs only a plain device-to-device copy of MIB MiB (3 launches), the
           reference against which hardware byte counters are scaled
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_F32_TFLOPS = 157.3       # MI355X published fp32 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("fa_kernels.hip", "fa_api.cpp", "fa_internal.h"):
        with open(os.path.join(ROOT, "online_softmax_fa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attention_flops(B, H, Nq, Nk, d, causal):
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f


def traffic_from_profile(workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_hbm_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, seconds):
    """Time the fp64 oracle on a bounded, evenly spread sample of query rows
    (all heads), with every host core this process may use."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    q, k, v = (x.float().numpy() for x in (w["q"], w["k"], w["v"]))
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    threads = len(os.sched_getaffinity(0))
    total_rows = B * H * N

    def row_flops(rows):
        i = rows % N
        keys = (i + 1) if w["causal"] else np.full_like(i, N)
        return float(np.sum(4.0 * d * keys))

    def timed(nrows):
        rows = np.linspace(0, total_rows - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        _, _, used = oracle.attn_fwd(q, k, v, w["scale"], causal=w["causal"], rows=rows,
                                     threads=threads)
        return time.perf_counter() - t0, row_flops(rows), used

    n = max(threads, 16)
    dt, fl, used = timed(n)
    while dt < 1.0 and n < total_rows:
        n = min(total_rows, n * 4)
        dt, fl, used = timed(n)
    if dt < seconds and n < total_rows:
        n = int(min(total_rows, n * seconds / max(dt, 1e-3)))
        dt, fl, used = timed(n)
    # the metric's flop count counts a causal run as half of the full square
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": "%d of %d query rows (evenly spaced over all heads), fp64 three-pass "
                  "oracle, %.1f s wall" % (n, total_rows, dt),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--block-n", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the attention kernel runs on a single MI355X and this "
              "build has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_fa_amd as fa
    from online_softmax_fa_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    fa.load_library()
    dev = torch.device("cuda:0")
    w = inputs.workload(args.workload)
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    log("workload %s: B=%d H=%d N=%d d=%d %s causal=%d" % (args.workload, B, H, N, d, w["dtype"],
                                                         w["causal"]))
    q, k, v = (x.to(dev) for x in (w["q"], w["k"], w["v"]))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)

    def step():
        fa.attention(q, k, v, scale=w["scale"], causal=w["causal"], block_n=args.block_n,
                     out=(o, lse))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = ev0.elapsed_time(ev1)
    ms = ms_total / args.steps
    log("timed %d steps: %.3f ms/step (events), %.3f ms/step (wall)" % (
        args.steps, ms, 1e3 * t_wall / args.steps))

    flops = attention_flops(B, H, N, N, d, w["causal"])
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_F32_TFLOPS
    props = torch.cuda.get_device_properties(dev)
    log("%.1f TFLOP/s = %.1f%% of %.0f TFLOP/s (%s, %d CUs)" % (
        tflops, 100 * tflops / peak, peak, props.name, props.multi_processor_count))

    traffic = traffic_from_profile(args.workload)
    result = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak, 1 MI355X, N=8192 d=128 causal",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {
            "workload": "%s: B=%d H=%d N_q=N_k=%d d=%d %s %s, Q/K/V ~ N(0,%g^2)" % (
                args.workload, B, H, N, d, w["dtype"], "causal" if w["causal"] else "non-causal",
                w["std"]),
            "B": B, "H": H, "N_q": N, "N_k": N, "d": d, "causal": bool(w["causal"]),
            "block_n": args.block_n or 64,
        },
        "pct_of_peak": round(100 * tflops / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of rows ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        log("cpu baseline: %s" % result["cpu_baseline"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
