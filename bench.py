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
  launch_ms  median and minimum of 20 steps timed one by one, after the
             timed region (`value` and ms_per_step are the mean of the K)
  counters   matrix-core busy %, vector issue %, LDS bank conflicts and HBM
             GB/s of the kernel, from the committed rocprofv3 summary
             (profiles/), while it was taken on the kernel code in the built
             library; else null
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload's rows, on this host's cores, in the same unit
  parity     the last launch's o and lse on those sample rows against the
             oracle's: max-abs and mean-abs of o, max-abs of lse, the bars
             and pass/fail
  peak_from_device  CUs x peak engine clock x 4096 (bf16 FLOP per CU per
             clock) as the device reports them, beside the published 2.5 PF

With --workload softmax (8192 rows of 8192 fp32 scores) a step is one
fa_softmax_rows call, reported as HBM GB/s of its compulsory bytes (the rows
read once and written once).

With --workload decode (8 sequences x 8 heads, one query each over 32768
keys) a step is one fa_fwd_splitkv call (split-key pass + merge, the
library's split count), and the line reports HBM GB/s: that workload is
bound by reading K and V once, so its roofline is the 8 TB/s HBM peak.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--block-n BN] [--splits S] [--no-cpu-baseline] [--cpu-seconds S]
       python bench.py --copy-calibration MIB
           runs only a plain device-to-device copy of MIB MiB (3 launches), the
           reference against which hardware byte counters are scaled
"""

import argparse
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_F32_TFLOPS = 157.3       # MI355X published fp32 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Kernels whose machine code decides each workload's counters and HBM
# traffic (substrings of their symbol names in the gfx950 code objects of
# libfa.so).  A stored counter summary is used only while that code is the
# code it was taken on: comments and unrelated kernels do not invalidate it,
# a change of source, compiler or flags that changes the code does.
PROFILED_KERNELS = {
    "headline": ("fa_fwd_bf16_kernelILi128ELi64ELi8ELb1ELb0E",),
    "long": ("fa_fwd_bf16_kernelILi128ELi64ELi8ELb0ELb0E",),
    "mid": ("fa_fwd_bf16_kernelILi64ELi64ELi4ELb1ELb0E",),
    "decode": ("fa_decode_bf16_kernelILi128E", "fa_merge_kernelILi128E"),
    "softmax": ("fa_softmax_rows_kernel",),
}
_BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _elf_sections(d):
    """[(name, addr, offset, size, type, link)] of a 64-bit little-endian ELF image."""
    shoff = struct.unpack_from("<Q", d, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    raw = [struct.unpack_from("<IIQQQQIIQQ", d, shoff + i * shentsize) for i in range(shnum)]
    stroff = raw[shstrndx][4]
    return [(d[stroff + r[0]: d.index(b"\0", stroff + r[0])].decode(), r[3], r[4], r[5], r[1], r[6])
            for r in raw]


def device_kernels(lib_path, arch="gfx950"):
    """{symbol name: machine code} of every function in lib_path's device
    code objects for arch (clang offload bundles in its .hip_fatbin section)."""
    with open(lib_path, "rb") as fh:
        d = fh.read()
    fat = next((d[o:o + n] for (nm, a, o, n, t, l) in _elf_sections(d) if nm == ".hip_fatbin"), b"")
    kernels = {}
    pos = fat.find(_BUNDLE_MAGIC)
    while pos >= 0:
        q = pos + len(_BUNDLE_MAGIC) + 8
        for _ in range(struct.unpack_from("<Q", fat, pos + len(_BUNDLE_MAGIC))[0]):
            off, size, idlen = struct.unpack_from("<QQQ", fat, q)
            ident = fat[q + 24: q + 24 + idlen].decode()
            q += 24 + idlen
            if not ident.endswith(arch):
                continue
            co = fat[pos + off: pos + off + size]
            secs = _elf_sections(co)
            for (nm, a, o, sz, t, link) in secs:
                if t != 2:                                   # SHT_SYMTAB
                    continue
                stro = secs[link][2]
                for k in range(sz // 24):
                    st_name, st_info, _, st_shndx, st_value, st_size = \
                        struct.unpack_from("<IBBHQQ", co, o + 24 * k)
                    if st_info & 0xF != 2 or st_size == 0:     # STT_FUNC
                        continue
                    name = co[stro + st_name: co.index(b"\0", stro + st_name)].decode()
                    sec = secs[st_shndx]
                    start = sec[2] + st_value - sec[1]
                    kernels[name] = co[start: start + st_size]
        pos = fat.find(_BUNDLE_MAGIC, pos + len(_BUNDLE_MAGIC))
    return kernels


_CODE_HASHES = {}


def kernel_code_hash(workload):
    """First 16 hex digits of the SHA-256 of the workload's kernels' names and
    machine code in the built libfa.so, or None if they cannot be read."""
    if workload not in _CODE_HASHES:
        try:
            ks = device_kernels(os.path.join(ROOT, "online_softmax_fa_amd", "libfa.so"))
            names = sorted(n for n in ks if any(p in n for p in PROFILED_KERNELS[workload]))
            h = hashlib.sha256()
            for n in names:
                h.update(n.encode())
                h.update(ks[n])
            _CODE_HASHES[workload] = h.hexdigest()[:16] if names else None
        except (OSError, KeyError, ValueError, struct.error, IndexError):
            _CODE_HASHES[workload] = None
    return _CODE_HASHES[workload]


def attention_flops(B, H, Nq, Nk, d, causal):
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f


def per_launch_ms(step, stream, torch, n=20):
    """Median and minimum of n steps timed one by one (an event pair around
    each, on the stream the kernels run on), after the timed region."""
    times = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return {"median": round(times[n // 2], 4), "min": round(times[0], 4), "launches": n}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def visible_pairs(Nq, lengths, causal):
    """(query, key) pairs of one head summed over sequences, with keys
    j < L visible and, under causality, j <= i."""
    total = 0
    for L in lengths:
        if not causal:
            total += Nq * L
        elif L >= Nq:
            total += Nq * (Nq + 1) // 2
        else:
            total += L * (L + 1) // 2 + (Nq - L) * L
    return total


def algorithmic_bytes(B, H, Nq, Nk, d, esz):
    """Q, K, V read once; O and lse written once."""
    return B * H * (2 * Nq * d * esz + 2 * Nk * d * esz + Nq * 4)


def traffic_from_profile(workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel code in the built library; else None."""
    path = os.path.join(ROOT, "profiles", "%s_hbm_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    code = kernel_code_hash(workload)
    if code is None or t.get("kernel_code_sha256_16") != code:
        return None
    return t.get("bytes_per_launch")


def counters_from_profile(workload):
    """Hardware counters of the dominant kernel from the committed rocprofv3
    summary (matrix-core busy %, vector issue %, LDS bank conflicts, HBM
    GB/s), if they were taken on the kernel code in the built library; else
    None."""
    path = os.path.join(ROOT, "profiles", "%s_counters.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    code = kernel_code_hash(workload)
    if code is None or t.get("kernel_code_sha256_16") != code:
        return None
    return {k: t[k] for k in ("mfma_busy_pct", "valu_issue_pct", "lds_bank_conflicts",
                              "exp2_per_mfma", "hbm_gb_per_s", "sustained_clock_ghz",
                              "cu_busy_pct") if k in t}


def cpu_baseline(w, seconds):
    """Time the fp64 oracle on a bounded, evenly spread sample of query rows
    (all heads), with every host core this process may use."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    q, k, v = (x.float().numpy() for x in (w["q"], w["k"], w["v"]))
    mask = None if w.get("mask") is None else w["mask"].numpy()
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    Nq = w["Nq"]
    threads = len(os.sched_getaffinity(0))
    total_rows = B * H * Nq
    hbm = w.get("bound") == "hbm"
    esz = 2 if w["dtype"] == "bf16" else 4

    def row_flops(rows):
        if hbm:   # the metric's unit: algorithmic bytes of the rows' heads, per row
            return float(len(rows)) * algorithmic_bytes(B, H, Nq, N, d, esz) / total_rows
        i = rows % Nq
        keys = (i + 1) if w["causal"] else np.full_like(i, N)
        return float(np.sum(4.0 * d * keys))

    def timed(nrows):
        rows = np.linspace(0, total_rows - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        o_ref, lse_ref, used = oracle.attn_fwd(q, k, v, w["scale"], causal=w["causal"],
                                               mask=mask, rows=rows, threads=threads)
        return time.perf_counter() - t0, row_flops(rows), used, (rows, o_ref, lse_ref)

    n = max(threads, 16)
    dt, fl, used, ref = timed(n)
    while dt < 1.0 and n < total_rows:
        n = min(total_rows, n * 4)
        dt, fl, used, ref = timed(n)
    if dt < seconds and n < total_rows:
        n = int(min(total_rows, n * seconds / max(dt, 1e-3)))
        dt, fl, used, ref = timed(n)
    # the metric's flop count counts a causal run as half of the full square
    return {
        "value": fl / dt / (1e9 if hbm else 1e12),
        "unit": "GB/s" if hbm else "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": "%d of %d query rows (evenly spaced over all heads), fp64 three-pass "
                  "oracle, %.1f s wall" % (n, total_rows, dt),
    }, ref


# Parity bars: O max-abs (and mean-abs for bf16) against the fp64 oracle, lse
# max-abs; rows with no visible key must be exactly o = 0, lse = -inf.
PARITY_BARS = {"f32": {"max_abs": 1e-5, "mean_abs": None, "lse_max_abs": 1e-3},
               "bf16": {"max_abs": 2e-2, "mean_abs": 2e-3, "lse_max_abs": 1e-3}}


def parity(o, lse, ref, dtype):
    """The GPU's o and lse (of the last launch, same inputs) on the oracle's
    sample rows against the oracle's fp64 values."""
    import numpy as np
    import torch
    rows, o_ref, lse_ref = ref
    d = o.shape[-1]
    idx = torch.from_numpy(rows).to(o.device)
    og = o.reshape(-1, d)[idx].float().cpu().numpy().astype(np.float64)
    lg = lse.reshape(-1)[idx].cpu().numpy().astype(np.float64)
    o_ref = o_ref.reshape(-1, d)
    dead = np.isneginf(lse_ref)
    live = ~dead
    bars = PARITY_BARS[dtype]
    out = {"rows": int(len(rows)), "rows_without_visible_key": int(dead.sum()),
           "bars": bars}
    ok = bool(np.all(og[dead] == 0.0) and np.all(np.isneginf(lg[dead])) and
              np.all(np.isfinite(og)) and np.all(np.isfinite(lg[live])))
    if live.any():
        err = np.abs(og[live] - o_ref[live])
        out["max_abs"] = float(err.max())
        out["mean_abs"] = float(err.mean())
        out["lse_max_abs"] = float(np.abs(lg[live] - lse_ref[live]).max())
        ok = ok and out["max_abs"] <= bars["max_abs"] and out["lse_max_abs"] <= bars["lse_max_abs"]
        if bars["mean_abs"] is not None:
            ok = ok and out["mean_abs"] <= bars["mean_abs"]
    out["pass"] = ok
    return out


def device_peak(torch, dev):
    """CUs x peak engine clock x 4096 bf16 FLOP per CU per clock (gfx950
    dense MFMA), from the device the bench runs on (HIP runtime attributes,
    through the runtime torch has loaded)."""
    import ctypes
    try:
        hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    except OSError:
        hip = ctypes.CDLL("libamdhip64.so")
    val = ctypes.c_int(0)
    idx = dev.index or 0

    def attr(a):    # hipDeviceAttributeClockRate = 5 (kHz), MultiprocessorCount = 63
        return val.value if hip.hipDeviceGetAttribute(ctypes.byref(val), a, idx) == 0 else 0

    khz, cus = attr(5), attr(63)
    if khz <= 0 or cus <= 0:
        return None
    return {"cus": cus, "clock_mhz": round(khz / 1e3, 1),
            "tflops": round(cus * khz * 1e3 * 4096 / 1e12, 1)}


def cpu_tiled(w, seconds):
    """The host-CPU tiled implementation of the same recurrence
    (libfa_cpu.so) on whole heads of the workload, as many as fit in about
    `seconds`, on every core this process may use; in the metric's unit."""
    import numpy as np
    import torch
    from online_softmax_fa_amd import cpu

    B, H, N, d, Nq = w["B"], w["H"], w["N"], w["d"], w["Nq"]
    bf16 = w["dtype"] == "bf16"
    threads = len(os.sched_getaffinity(0))

    def arr(t, nh):
        x = t.reshape(B * H, -1, d)[:nh].contiguous()
        return x.view(torch.int16).numpy().view(np.uint16) if bf16 else x.numpy()

    # with key-padding masks, heads of the first sequence only (one mask row)
    mask = None if w.get("mask") is None else w["mask"][:1].numpy()
    max_heads = B * H if mask is None else H

    def timed(nh):
        q, k, v = (arr(w[x], nh).reshape(1, nh, -1, d) for x in ("q", "k", "v"))
        t0 = time.perf_counter()
        _, _, used = cpu.attention_cpu(q, k, v, w["scale"], w["causal"], mask, threads,
                                       dtype="bf16" if bf16 else "f32")
        return time.perf_counter() - t0, used

    nh = 1
    dt, used = timed(nh)
    if dt < seconds and nh < max_heads:
        nh = int(min(max_heads, max(1, seconds / max(dt, 1e-3))))
        dt, used = timed(nh)
    esz = 2 if bf16 else 4
    if w.get("bound") == "hbm":
        value, unit = nh * algorithmic_bytes(1, 1, Nq, N, d, esz) / dt / 1e9, "GB/s"
    else:
        value, unit = nh * attention_flops(1, 1, Nq, N, d, w["causal"]) / dt / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": int(used), "kind": "cpu_tiled",
            "cpu": cpu_model(),
            "sample": "%d of %d heads, libfa_cpu.so (the same recurrence, cache-tiled and "
                      "vectorized on the host), %.1f s wall" % (nh, B * H, dt)}


def softmax_cpu_baseline(s, seconds):
    """The fp64 oracle's three-pass softmax on evenly spaced rows, one core
    (the oracle's row entry point is single-threaded), in GB/s of the rows'
    compulsory bytes."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    a = s.float().numpy()
    rows, n = a.shape
    nb = 2 * n * s.element_size()
    t0 = time.perf_counter()
    done = 0
    for r in np.linspace(0, rows - 1, rows).astype(np.int64):
        oracle.softmax_row(a[r].astype(np.float64))
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done * nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "%d of %d rows (evenly spaced), fp64 three-pass oracle, %.1f s wall" % (
                done, rows, dt)}


def bench_softmax(args, torch, fa, inputs):
    dev = torch.device("cuda:0")
    w = inputs.row_workload(args.workload)
    rows, n = w["rows"], w["n"]
    log("workload %s: %d rows x %d %s" % (args.workload, rows, n, w["dtype"]))
    s = w["s"].to(dev)
    p = torch.empty_like(s)

    def step():
        fa.softmax_rows(s, out=p)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    launch_ms = per_launch_ms(step, stream, torch)
    nbytes = 2 * rows * n * s.element_size() + 2 * rows * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("%.3f ms/step, %.1f GB/s = %.1f%% of %.0f GB/s" % (ms, gbs, 100 * gbs / PEAK_HBM_GBS,
                                                          PEAK_HBM_GBS))
    result = {
        "metric": "online-softmax over score rows, HBM GB/s of the compulsory bytes, 1 MI355X",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": "%s: %d rows x %d %s scores ~ N(0,%g^2)" % (
            args.workload, rows, n, w["dtype"], w["std"]), "rows": rows, "n": n},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "launch_ms": launch_ms,
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profile(args.workload)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = softmax_cpu_baseline(w["s"], args.cpu_seconds)
        log("cpu baseline: %s" % result["cpu_baseline"])
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--block-n", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0,
                    help="decode: split count (0: the library's choice)")
    ap.add_argument("--kv-lengths", action="store_true",
                    help="key-padding prefix masks: per-sequence key lengths drawn uniformly "
                         "from [N_k/2, N_k] (seed: the workload's + 1000)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the attention kernel runs on a single MI355X and this "
              "library has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
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
    if args.workload in inputs.ROW_WORKLOADS:
        return bench_softmax(args, torch, fa, inputs)
    dev = torch.device("cuda:0")
    w = inputs.workload(args.workload)
    B, H, N, d, Nq = w["B"], w["H"], w["N"], w["d"], w["Nq"]
    split = args.workload == "decode"
    w["bound"] = "hbm" if split else "mfma"
    log("workload %s: B=%d H=%d N_q=%d N_k=%d d=%d %s causal=%d" % (
        args.workload, B, H, Nq, N, d, w["dtype"], w["causal"]))
    q, k, v = (x.to(dev) for x in (w["q"], w["k"], w["v"]))
    mask_d, lens = None, None
    if args.kv_lengths:
        lens = inputs.kv_lengths(B, N, inputs.WORKLOADS[args.workload]["seed"] + 1000)
        w["mask"] = inputs.prefix_mask(lens, N)
        mask_d = w["mask"].to(dev)
        log("key lengths per sequence: %s" % lens.tolist())
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)

    if split:
        ns = args.splits or fa.fa_splitkv_splits(B, H, Nq, N, d, w["causal"])
        ws = torch.empty(fa.fa_splitkv_workspace_bytes(B, H, Nq, d, ns), dtype=torch.uint8,
                         device=dev)
        log("split-key path: %d splits, workspace %d bytes" % (ns, ws.numel()))

        def step():
            fa.attention_splitkv(q, k, v, scale=w["scale"], causal=w["causal"], num_splits=ns,
                                 kv_len_mask=mask_d, out=(o, lse), workspace=ws)
    else:
        def step():
            fa.attention(q, k, v, scale=w["scale"], causal=w["causal"], block_n=args.block_n,
                         kv_len_mask=mask_d, out=(o, lse))

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
    launch_ms = per_launch_ms(step, stream, torch)
    log("timed %d steps: %.3f ms/step (events), %.3f ms/step (wall)" % (
        args.steps, ms, 1e3 * t_wall / args.steps))

    flops = attention_flops(B, H, Nq, N, d, w["causal"])
    tflops = flops / (ms * 1e-3) / 1e12
    esz = 2 if w["dtype"] == "bf16" else 4
    nbytes = algorithmic_bytes(B, H, Nq, N, d, esz)
    gbs = nbytes / (ms * 1e-3) / 1e9
    props = torch.cuda.get_device_properties(dev)
    if split:
        value, unit, peak, achieved = gbs, "GB/s", PEAK_HBM_GBS, gbs
        metric = "split-key attention fwd (decode), HBM GB/s of the algorithmic bytes, 1 MI355X"
        log("%.1f GB/s = %.1f%% of %.0f GB/s; %.2f TFLOP/s (%s, %d CUs)" % (
            gbs, 100 * gbs / peak, peak, tflops, props.name, props.multi_processor_count))
    else:
        peak = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_F32_TFLOPS
        value, unit, achieved = tflops, "TFLOP/s", tflops
        if args.workload == "headline":
            metric = "attention fwd TFLOP/s and % of bf16 MFMA peak, 1 MI355X, N=8192 d=128 causal"
        else:
            metric = "attention fwd TFLOP/s and %% of %s MFMA peak, 1 MI355X, N=%d d=%d %s" % (
                w["dtype"], N, d, "causal" if w["causal"] else "non-causal")
        dpeak = device_peak(torch, dev)
        if dpeak:
            log("bf16 dense peak from the device: %d CUs x %.0f MHz x 4096 FLOP/clk = %.1f "
                "TFLOP/s (published: 2500)" % (dpeak["cus"], dpeak["clock_mhz"], dpeak["tflops"]))
        log("%.1f TFLOP/s = %.1f%% of %.0f TFLOP/s (%s, %d CUs)" % (
            tflops, 100 * tflops / peak, peak, props.name, props.multi_processor_count))

    traffic = traffic_from_profile(args.workload)
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
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
            "workload": "%s: B=%d H=%d N_q=%d N_k=%d d=%d %s %s, Q/K/V ~ N(0,%g^2)" % (
                args.workload, B, H, Nq, N, d, w["dtype"],
                "causal" if w["causal"] else "non-causal", w["std"]),
            "B": B, "H": H, "N_q": Nq, "N_k": N, "d": d, "causal": bool(w["causal"]),
            "block_n": args.block_n or 64,
        },
        "pct_of_peak": round(100 * value / peak, 2),
        "launch_ms": launch_ms,
        "tflops": round(tflops, 3),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {
            "bound": "hbm" if split else "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "counters": counters_from_profile(args.workload),
        "cpu_baseline": None,
        "parity": None,
    }
    if not split:
        result["peak_from_device"] = dpeak
        cnt = result["counters"] or {}
        if "sustained_clock_ghz" in cnt and dpeak:
            # the matrix-core ceiling at the clock the chip held under this load
            result["peak_at_sustained_clock"] = round(
                dpeak["cus"] * cnt["sustained_clock_ghz"] * 1e9 * 4096 / 1e12, 1)
    if split:
        result["config"]["splits"] = ns
    if lens is not None:
        # the metric counts every (query, key) pair; the visible ones are fewer
        vis = visible_pairs(Nq, lens.tolist(), w["causal"]) * H
        result["config"]["kv_lengths"] = lens.tolist()
        result["effective_tflops"] = round(4.0 * d * vis / (ms * 1e-3) / 1e12, 3)
        log("effective: %.1f TFLOP/s over the visible (query, key) pairs" %
            result["effective_tflops"])
        if not split:
            # the kernel's algorithmic work is the visible pairs' products
            eff = result["effective_tflops"]
            result["roofline"]["achieved"] = eff
            result["roofline"]["frac"] = round(eff / peak, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of rows ...")
        result["cpu_baseline"], ref = cpu_baseline(w, args.cpu_seconds)
        log("cpu baseline: %s" % result["cpu_baseline"])
        # the oracle's rows are the parity check of the last launch's output
        result["parity"] = parity(o, lse, ref, w["dtype"])
        log("parity against the fp64 oracle: %s" % result["parity"])
        log("timing the host-CPU tiled implementation on whole heads ...")
        result["cpu_tiled"] = cpu_tiled(w, args.cpu_seconds / 3)
        log("cpu tiled: %s" % result["cpu_tiled"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
