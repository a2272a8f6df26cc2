"""The Python binding refuses caller-supplied outputs that do not match what
the kernels write, before anything is enqueued: the C layer sees only device
pointers, so a smaller or differently typed buffer would be written past its
end.  Each bad output raises FaError and leaves every buffer as it was."""

import pytest
import torch

import online_softmax_fa_amd as fa
from online_softmax_fa_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def _qkv(dtype="f32", B=1, H=2, N=70, d=64):
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, seed=8100, dtype=dtype)
    return q.to(DEV), k.to(DEV), v.to(DEV)


def _bad_outs(q):
    B, H, Nq, d = q.shape
    other = torch.bfloat16 if q.dtype == torch.float32 else torch.float32
    good_o = torch.full_like(q, 7.0)
    good_l = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device=DEV)
    return [
        ("o dtype", (torch.full(q.shape, 7.0, dtype=other, device=DEV), good_l)),
        ("o shape", (torch.full((B, H, Nq - 1, d), 7.0, dtype=q.dtype, device=DEV), good_l)),
        ("o not contiguous", (torch.full((B, H, d, Nq), 7.0, dtype=q.dtype,
                                         device=DEV).transpose(2, 3), good_l)),
        ("o on the host", (torch.full(q.shape, 7.0, dtype=q.dtype), good_l)),
        ("lse dtype", (good_o, torch.full((B, H, Nq), 7.0, dtype=torch.float64, device=DEV))),
        ("lse shape", (good_o, torch.full((B, H, Nq + 1), 7.0, dtype=torch.float32,
                                          device=DEV))),
    ]


def _unchanged(out):
    torch.cuda.synchronize()
    return all(bool((t.float() == 7.0).all()) for t in out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_rejects_bad_outputs(dtype):
    q, k, v = _qkv(dtype)
    for what, out in _bad_outs(q):
        with pytest.raises(fa.FaError):
            fa.attention(q, k, v, out=out)
        assert _unchanged(out), what
        with pytest.raises(fa.FaError):
            fa.attention_splitkv(q, k, v, num_splits=2, out=out)
        assert _unchanged(out), what


def test_softmax_rows_rejects_bad_outputs():
    s = torch.randn(4, 100, device=DEV)
    for bad in (torch.full((4, 99), 7.0, device=DEV),
                torch.full((4, 100), 7.0, dtype=torch.bfloat16, device=DEV),
                torch.full((100, 4), 7.0, device=DEV).t()):
        with pytest.raises(fa.FaError):
            fa.softmax_rows(s, out=bad)
        assert _unchanged([bad])


def test_merge_states_rejects_bad_outputs():
    n_parts, rows, d = 3, 10, 64
    m = torch.zeros(n_parts, rows, device=DEV)
    l = torch.ones(n_parts, rows, device=DEV)
    acc = torch.zeros(n_parts, rows, d, device=DEV)
    lse = torch.full((rows,), 7.0, device=DEV)
    for bad in ((torch.full((rows, d + 1), 7.0, device=DEV), lse),
                (torch.full((rows, d), 7.0, device=DEV), torch.full((rows - 1,), 7.0, device=DEV))):
        with pytest.raises(fa.FaError):
            fa.merge_states(m, l, acc, 0.125, out=bad)
        assert _unchanged(bad)


def test_good_outputs_still_accepted():
    q, k, v = _qkv("bf16")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    o2, lse2 = fa.attention(q, k, v, out=(o, lse))
    assert o2 is o and lse2 is lse
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
