"""The C-ABI boundary, checked without a GPU: the library loads, exports every
entry point include/fa.h declares, rejects bad arguments with the documented
codes before touching any device, and stays independent of the oracle."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

import online_softmax_fa_amd as fa  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    return fa.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["fa_fwd", "fa_fwd_ex", "fa_fwd_splitkv",
                                     "fa_fwd_splitkv_noalloc", "fa_merge_states",
                                     "fa_query_tile_rows", "fa_softmax_rows", "fa_splitkv_splits",
                                     "fa_splitkv_workspace_bytes", "fa_strerror"]


def test_query_tile_rows(lib):
    """Rows per workgroup: 128 or 256, fixed by the arguments alone (no device
    needed); 256 only for bf16 with d = 128, 64-key tiles and enough
    workgroups (the headline and long-context shapes); bad arguments give
    their status."""
    F32, BF16 = fa.FA_DTYPE_F32, fa.FA_DTYPE_BF16
    q = lib.fa_query_tile_rows
    for dtype in (F32, BF16):
        for d in (64, 128):
            for nq in (1, 128, 129, 8192):
                for bn in (0, 16, 32, 64, 128):
                    for causal in (0, 1):
                        assert q(dtype, 2, 32, nq, d, bn, causal) in (128, 256)
                assert q(dtype, 2, 32, nq, d, 0, 1) == q(dtype, 2, 32, nq, d, 64, 1)
    assert q(BF16, 2, 32, 8192, 128, 64, 1) == 256          # headline, causal
    assert q(BF16, 1, 8, 32768, 128, 64, 0) == 256          # long context, non-causal
    assert q(BF16, 2, 16, 4096, 128, 64, 1) == 256          # causal, 2 workgroups per CU
    assert q(BF16, 1, 8, 8192, 128, 64, 1) == 128           # causal, too few workgroups
    assert q(BF16, 1, 4, 8192, 128, 64, 0) == 128           # non-causal, too few workgroups
    assert q(BF16, 2, 32, 8192, 64, 64, 1) == 128           # d = 64
    assert q(BF16, 2, 32, 8192, 128, 32, 1) == 128          # other tile sizes
    assert q(BF16, 256, 8, 128, 128, 64, 0) == 128          # N_q <= 128
    assert q(F32, 2, 32, 8192, 128, 64, 1) == 128           # fp32 kernel
    assert q(BF16, 1, 1, 0, 64, 64, 0) == fa.FA_ERR_SHAPE
    assert q(BF16, 0, 1, 8, 64, 64, 0) == fa.FA_ERR_SHAPE
    assert q(BF16, 1, 1, 8, 96, 64, 0) == fa.FA_ERR_HEAD_DIM
    assert q(7, 1, 1, 8, 64, 64, 0) == fa.FA_ERR_DTYPE
    assert q(BF16, 1, 1, 8, 64, 48, 0) == fa.FA_ERR_TILE


def test_header_compiles_as_c_and_cxx(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "fa.h"\nint main(void){fa_opts o={0,0,0,0,0,0};(void)o;'
                   'size_t n=fa_splitkv_workspace_bytes(1,1,1,64,1);(void)n;'
                   'return fa_fwd(0,0,0,0,0,1,1,1,1,64,1.0f,0,0,FA_DTYPE_BF16,0)==FA_ERR_NULL?0:1;}\n')
    for comp, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        subprocess.run([comp, std, "-fsyntax-only", "-Wall", "-Werror", "-I",
                        os.path.join(ROOT, "include"), "-x", "c" if comp == "gcc" else "c++",
                        str(src)], check=True)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (fa_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_strerror_covers_every_code(lib):
    for code in range(0, -14, -1):
        s = fa.fa_strerror(code)
        assert s and s != "unknown status code", code
    assert fa.fa_strerror(-99) == "unknown status code"


FAKE = 0x10000          # never dereferenced: validation fails first
FAKE2 = 0x20000000
FAKE3 = 0x40000000
FAKE4 = 0x60000000
FAKE5 = 0x80000000


def _call(q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5, B=1, H=1, Nq=8, Nk=8, d=64, scale=0.125,
          causal=0, mask=None, dtype=1, block_n=0, trace=None, tb=0, th=0, trow=0):
    lib = fa.load_library()
    opts = fa.fa_opts(block_n, 0, trace, tb, th, trow)
    return lib.fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, mask, dtype, None,
                         ctypes.byref(opts))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(k=None), fa.FA_ERR_NULL), (dict(v=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=-1), fa.FA_ERR_SHAPE), (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(Nk=0), fa.FA_ERR_SHAPE), (dict(B=1 << 20, H=1 << 20, Nq=1 << 20), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM), (dict(d=256), fa.FA_ERR_HEAD_DIM),
    (dict(dtype=2), fa.FA_ERR_DTYPE), (dict(dtype=-1), fa.FA_ERR_DTYPE),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=-0.5), fa.FA_ERR_SCALE),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE), (dict(scale=float("inf")), fa.FA_ERR_SCALE),
    (dict(block_n=48), fa.FA_ERR_TILE), (dict(block_n=256), fa.FA_ERR_TILE),
    (dict(o=FAKE), fa.FA_ERR_ALIAS), (dict(lse=FAKE3 + 16), fa.FA_ERR_ALIAS),
    (dict(mask=FAKE4 + 1), fa.FA_ERR_ALIAS),
    (dict(trace=0x90000000, tb=1), fa.FA_ERR_ARG), (dict(trace=0x90000000, th=-1), fa.FA_ERR_ARG),
    (dict(trace=0x90000000, trow=8), fa.FA_ERR_ARG), (dict(trace=FAKE4 + 8), fa.FA_ERR_ALIAS),
    (dict(q=FAKE + 8), fa.FA_ERR_ALIGN), (dict(k=FAKE2 + 2), fa.FA_ERR_ALIGN),
    (dict(v=FAKE3 + 4), fa.FA_ERR_ALIGN), (dict(o=FAKE4 + 8), fa.FA_ERR_ALIGN),
    (dict(lse=FAKE5 + 2), fa.FA_ERR_ALIGN), (dict(trace=0x90000008), fa.FA_ERR_ALIGN),
])
def test_argument_errors_before_any_device_work(lib, kw, code):
    assert _call(**kw) == code


def test_valid_arguments_without_gpu_report_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call() == fa.FA_ERR_DEVICE
    assert _call(trace=0x90000000, tb=0, th=0, trow=7) == fa.FA_ERR_DEVICE
    assert _split() == fa.FA_ERR_DEVICE
    assert _merge() == fa.FA_ERR_DEVICE
    assert _noalloc() == fa.FA_ERR_DEVICE
    assert lib.fa_splitkv_splits(1, 8, 1, 32768, 128, 0) == fa.FA_ERR_DEVICE


WS = 0xA0000000


def _split(B=1, H=2, Nq=8, Nk=8, d=64, ns=3, ws=WS, ws_bytes=None, q=FAKE, o=FAKE4):
    lib = fa.load_library()
    if ws_bytes is None:
        ws_bytes = lib.fa_splitkv_workspace_bytes(B, H, Nq, d, ns if 1 <= ns <= 256 else 1)
    return lib.fa_fwd_splitkv(q, FAKE2, FAKE3, o, FAKE5, B, H, Nq, Nk, d, 0.125, 0, None, 1, ns,
                              ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(B=0), fa.FA_ERR_SHAPE), (dict(d=80), fa.FA_ERR_HEAD_DIM),
    (dict(ns=0), fa.FA_ERR_ARG), (dict(ns=257), fa.FA_ERR_ARG), (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=64), fa.FA_ERR_WORKSPACE), (dict(ws=WS + 4), fa.FA_ERR_WORKSPACE),
    (dict(ws=FAKE4 - 16), fa.FA_ERR_ALIAS), (dict(ws=FAKE), fa.FA_ERR_ALIAS),
])
def test_splitkv_argument_errors(lib, kw, code):
    assert _split(**kw) == code


def _noalloc(B=1, H=2, Nq=8, Nk=8, d=64, ns=3, q=FAKE, o=FAKE4, lse=FAKE5):
    lib = fa.load_library()
    return lib.fa_fwd_splitkv_noalloc(q, FAKE2, FAKE3, o, lse, B, H, Nq, Nk, d, 0.125, 0, None, 1,
                                      ns, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(B=0), fa.FA_ERR_SHAPE), (dict(d=80), fa.FA_ERR_HEAD_DIM),
    (dict(ns=0), fa.FA_ERR_ARG), (dict(ns=257), fa.FA_ERR_ARG), (dict(o=FAKE), fa.FA_ERR_ALIAS),
    (dict(lse=FAKE5 + 2), fa.FA_ERR_ALIGN),
    # partial states of 2*16*1024 rows x 16 parts x (128 + 2) floats: 272 MB > 32 MiB
    (dict(B=2, H=16, Nq=1024, Nk=1024, d=128, ns=16), fa.FA_ERR_SCRATCH),
])
def test_splitkv_noalloc_argument_errors(lib, kw, code):
    """The no-alloc split-key entry point checks what fa_fwd_splitkv checks
    (no workspace), and rejects partial states beyond its 32 MiB scratch, all
    before touching a device."""
    assert _noalloc(**kw) == code


def test_splitkv_noalloc_scratch_limit_is_the_workspace_size(lib):
    """The largest request that fits is the one whose fa_fwd_splitkv workspace
    is at most 32 MiB."""
    import torch
    limit = 32 << 20
    d, ns = 128, 16
    rows_max = max(r for r in range(1, 5000) if lib.fa_splitkv_workspace_bytes(1, 1, r, d, ns) <= limit)
    assert lib.fa_splitkv_workspace_bytes(1, 1, rows_max + 1, d, ns) > limit
    assert _noalloc(B=1, H=1, Nq=rows_max + 1, Nk=64, d=d, ns=ns) == fa.FA_ERR_SCRATCH
    if not torch.cuda.is_available():
        assert _noalloc(B=1, H=1, Nq=rows_max, Nk=64, d=d, ns=ns) == fa.FA_ERR_DEVICE


def test_splitkv_workspace_bytes_follow_the_documented_layout(lib):
    """m and l: float[S][rows] each; acc: float[S][rows][d] from the next
    multiple of 256 bytes."""
    for (B, H, Nq, d, S) in ((1, 8, 1, 128, 128), (2, 3, 5, 64, 7), (1, 1, 1, 64, 1)):
        rows = B * H * Nq
        acc_off = (2 * S * rows * 4 + 255) // 256 * 256
        assert lib.fa_splitkv_workspace_bytes(B, H, Nq, d, S) == acc_off + S * rows * d * 4
    for bad in ((0, 1, 1, 64, 1), (1, 1, 1, 96, 1), (1, 1, 1, 64, 0), (1, 1, 1, 64, 257)):
        assert lib.fa_splitkv_workspace_bytes(*bad) == 0


def _merge(m=FAKE, l=FAKE2, acc=FAKE3, n=4, rows=10, d=64, scale=0.5, o=FAKE4, lse=FAKE5, dt=1):
    return fa.load_library().fa_merge_states(m, l, acc, n, rows, d, scale, o, lse, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(m=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL), (dict(rows=0), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_HEAD_DIM), (dict(dt=3), fa.FA_ERR_DTYPE),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE), (dict(n=0), fa.FA_ERR_ARG),
    (dict(o=FAKE2 + 64), fa.FA_ERR_ALIAS), (dict(lse=FAKE3 + 4), fa.FA_ERR_ALIAS),
    (dict(lse=FAKE4 + 64), fa.FA_ERR_ALIAS),
    (dict(acc=FAKE3 + 4), fa.FA_ERR_ALIGN), (dict(o=FAKE4 + 8), fa.FA_ERR_ALIGN),
    (dict(m=FAKE + 2), fa.FA_ERR_ALIGN), (dict(lse=FAKE5 + 1), fa.FA_ERR_ALIGN),
])
def test_merge_argument_errors(lib, kw, code):
    assert _merge(**kw) == code


def _softmax(s=FAKE, p=FAKE2, m=FAKE3, l=FAKE4, rows=10, n=100, dt=0):
    return fa.load_library().fa_softmax_rows(s, p, m, l, rows, n, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(s=None), fa.FA_ERR_NULL), (dict(p=None), fa.FA_ERR_NULL), (dict(rows=0), fa.FA_ERR_SHAPE),
    (dict(n=-1), fa.FA_ERR_SHAPE), (dict(rows=1 << 40, n=1 << 40), fa.FA_ERR_SHAPE),
    (dict(dt=5), fa.FA_ERR_DTYPE), (dict(p=FAKE + 4), fa.FA_ERR_ALIAS),
    (dict(m=FAKE + 40), fa.FA_ERR_ALIAS), (dict(l=FAKE2 + 8), fa.FA_ERR_ALIAS),
    (dict(l=FAKE3 + 4), fa.FA_ERR_ALIAS),
    (dict(s=FAKE + 2), fa.FA_ERR_ALIGN), (dict(s=FAKE + 1, dt=1), fa.FA_ERR_ALIGN),
    (dict(p=FAKE2 + 6), fa.FA_ERR_ALIGN), (dict(m=FAKE3 + 2), fa.FA_ERR_ALIGN),
])
def test_softmax_argument_errors(lib, kw, code):
    assert _softmax(**kw) == code


def test_softmax_valid_arguments_without_gpu(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _softmax() == fa.FA_ERR_DEVICE
    assert _softmax(p=FAKE) == fa.FA_ERR_DEVICE            # in place
    assert _softmax(m=None, l=None) == fa.FA_ERR_DEVICE


def test_binding_raises_with_the_message(lib):
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_ex(FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 1, 8, 8, 100, 0.125, 0, None, 1, None)
    assert e.value.code == fa.FA_ERR_HEAD_DIM and "64 or 128" in str(e.value)


def test_product_path_is_independent_of_the_oracle():
    """Neither the library sources nor the binding refer to the oracle, and the
    built library links no oracle code."""
    pkg = os.path.join(ROOT, "online_softmax_fa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "ref_attn" not in text and "libfaref" not in text, f
    out = subprocess.run(["objdump", "-p", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "faref" not in out


def test_every_kernel_has_its_host_stub():
    """A kernel whose host-side stub was not emitted shows up as an undefined
    symbol and would only fail when the library is loaded on the GPU."""
    out = subprocess.run(["nm", "-C", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "fa::" in l]
    assert not undefined, undefined
    defined = [l for l in out.splitlines() if "fa::fa_fwd_" in l and "_kernel<" in l]
    assert len(defined) >= 64, len(defined)
    merge = [l for l in out.splitlines() if "__device_stub__fa_merge_kernel<" in l]
    assert len(merge) == 4, merge
    sm = [l for l in out.splitlines() if "__device_stub__fa_softmax_rows_kernel<" in l]
    assert len(sm) == 6, sm


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with status 2 and says
    so, before touching any device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("fa_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_reads_kernel_code_from_the_library():
    """bench.py keys the committed counter summaries by the machine code of
    each workload's kernels, read from the gfx950 code objects in libfa.so:
    every profiled workload finds its kernels there, and the hash depends on
    the code alone."""
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    b = _bench_module()
    ks = b.device_kernels(fa.LIB_PATH)
    assert ks, "no gfx950 device functions found in libfa.so"
    for workload, patterns in b.PROFILED_KERNELS.items():
        for p in patterns:
            assert any(p in n for n in ks), (workload, p)
        h = b.kernel_code_hash(workload)
        assert h is not None and len(h) == 16 and int(h, 16) >= 0
    # every kernel is whole machine code: a multiple of the 4-byte instruction unit
    assert all(len(code) % 4 == 0 and len(code) > 0 for code in ks.values())
    assert b.kernel_code_hash("headline") != b.kernel_code_hash("long")
