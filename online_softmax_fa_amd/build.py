"""Compile libfa.so for gfx950 with hipcc, in-tree.

Usage: python -m online_softmax_fa_amd.build   (or __graft_entry__.build())
"""

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
SOURCES = [os.path.join(_HERE, "csrc", f)
           for f in ("fa_kernels.hip", "fa_decode.hip", "fa_softmax.hip", "fa_noalloc.hip",
                     "fa_api.cpp")]
OUT = os.path.join(_HERE, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _filter(stderr):
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    return "\n".join(x for x in stderr.splitlines() if noise not in x)


def build(verbose=False):
    """Compile every source to an object in parallel, then link libfa.so."""
    tmp = OUT + ".tmp%d" % os.getpid()
    inc = ["-I", os.path.join(_ROOT, "include"), "-I", os.path.join(_HERE, "csrc")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in SOURCES:
        obj = "%s.%s.o" % (tmp, os.path.basename(src))
        cmd = [HIPCC] + compile_flags + inc + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        _, err = pr.communicate()
        err = _filter(err)
        if pr.returncode != 0:
            failed.append("%s (%d):\n%s" % (src, pr.returncode, err))
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    try:
        if failed:
            raise RuntimeError("hipcc failed: " + "\n".join(failed))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed (%d):\n%s" % (r.returncode, _filter(r.stderr)))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, OUT)
    return OUT


CPU_SOURCE = os.path.join(_HERE, "csrc", "fa_cpu.cpp")
CPU_OUT = os.path.join(_HERE, "libfa_cpu.so")


def build_cpu(verbose=False):
    """Compile libfa_cpu.so, the host-CPU implementation, with g++ (OpenMP;
    no fast-math: the kernel relies on IEEE -inf and rounding)."""
    tmp = CPU_OUT + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O3", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-I", os.path.join(_ROOT, "include"), CPU_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed (%d):\n%s" % (r.returncode, r.stderr))
    os.replace(tmp, CPU_OUT)
    return CPU_OUT


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_cpu(verbose=True))
