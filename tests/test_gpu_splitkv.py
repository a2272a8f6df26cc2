"""GPU parity of the split-key path and of the partial-state merge.

fa_fwd_splitkv cuts every row's keys into ranges whose partial states are
merged; the result must match the fp64 oracle at the same bars as fa_fwd
("The math of FlashAttention", "Proof of exactness": block size and order never
enter the result).  The partial states left in the workspace are checked
against the oracle's partial_state of each key range, and fa_merge_states
against the oracle's merge_states and, end to end, against the three-pass
oracle over all keys.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.online import merge_states, partial_state
from online_softmax_fa_amd import inputs
import online_softmax_fa_amd as fa
from _parity import compare, run_oracle, say, to_np32

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()


def run_split(q, k, v, scale, causal=False, mask=None, num_splits=None, workspace=None):
    qd, kd, vd = (x.contiguous().to(DEV) for x in (q, k, v))
    md = None if mask is None else mask.contiguous().to(DEV)
    o, lse = fa.attention_splitkv(qd, kd, vd, scale=scale, causal=causal, kv_len_mask=md,
                                  num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy()


_ORACLE = {}


def _adv_ref(case):
    if case not in _ORACLE:
        q, k, v = inputs.adversarial(dtype="f32")
        mask, causal = inputs.adversarial_cases()[case]
        _ORACLE[case] = run_oracle(q, k, v, inputs.ADV_SCALE, causal=causal, mask=mask)
    return _ORACLE[case]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64])
def test_splitkv_adversarial(dtype, splits):
    """Exact-score heads (maximum in the last tile, in the first, a jump that
    underflows alpha, maxima straddling ln FLT_MAX) with masks; 16 key tiles,
    so 64 splits leave most ranges empty."""
    q, k, v = inputs.adversarial(dtype=dtype)
    cases = inputs.adversarial_cases()
    for name in ("nomask", "bern30", "mask_max_keys", "causal_prefix_masked", "all_masked"):
        mask, causal = cases[name]
        say("adv %s splits=%d %s" % (dtype, splits, name))
        o, lse = run_split(q, k, v, inputs.ADV_SCALE, causal=causal, mask=mask, num_splits=splits)
        o_ref, lse_ref = _adv_ref(name)
        compare(o, lse, o_ref, lse_ref, dtype, what="%s s%d" % (name, splits))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 63), (1, 4099), (5, 1000), (33, 2049)])
def test_splitkv_decode_shapes(d, Nq, Nk):
    """Few queries over many keys, ragged key tails, per-batch key lengths and
    a batch whose keys are all masked; the library's split choice and two
    explicit ones."""
    B, H = 3, 2
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=2100 + Nq + Nk, dtype="bf16")
    lens = inputs.kv_lengths(B, Nk, seed=2200 + Nk, lo=1)
    mask = inputs.prefix_mask(lens, Nk)
    mask[2] = 0
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, mask=mask)
    for splits in (None, 2, 13):
        say("decode d=%d Nq=%d Nk=%d splits=%s" % (d, Nq, Nk, splits))
        o, lse = run_split(q, k, v, scale, mask=mask, num_splits=splits)
        compare(o, lse, o_ref, lse_ref, "bf16", what="splits %s" % splits)


@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_single_row_causal(d):
    """One query row under top-left causality sees key 0 alone, whatever the
    key count and split."""
    B, H, Nk = 2, 3, 1000
    q, k, v = inputs.gaussian_qkv(B, H, 1, Nk, d, seed=2250 + d, dtype="bf16")
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=True)
    for splits in (None, 1, 3):
        say("single causal row d=%d splits=%s" % (d, splits))
        o, lse = run_split(q, k, v, scale, causal=True, num_splits=splits)
        compare(o, lse, o_ref, lse_ref, "bf16", what="causal row splits %s" % splits)


@pytest.mark.parametrize("splits", [3, 5])
def test_splitkv_causal_prefill(splits):
    """Causal rows over key ranges: query tiles near the top have fewer tiles
    than splits, so some of their ranges are empty."""
    q, k, v = inputs.gaussian_qkv(1, 2, 700, 700, 128, seed=2300, dtype="bf16")
    scale = inputs.default_scale(128)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=True)
    o, lse = run_split(q, k, v, scale, causal=True, num_splits=splits)
    compare(o, lse, o_ref, lse_ref, "bf16", what="causal splits %d" % splits)


def test_splitkv_decode_workload_full_size():
    """The decode workload at its full size and the library's split choice
    (the configuration the bench times), every row against the oracle."""
    w = inputs.workload("decode")
    ns = fa.fa_splitkv_splits(w["B"], w["H"], w["Nq"], w["N"], w["d"], False)
    say("decode B=%d H=%d Nk=%d splits=%d" % (w["B"], w["H"], w["N"], ns))
    o, lse = run_split(w["q"], w["k"], w["v"], w["scale"], num_splits=ns)
    o_ref, lse_ref = run_oracle(w["q"], w["k"], w["v"], w["scale"])
    compare(o, lse, o_ref, lse_ref, "bf16", what="decode")


@pytest.mark.parametrize("dtype,Nq,d", [("f32", 3, 64), ("bf16", 1, 64), ("bf16", 1, 128)])
def test_splitkv_workspace_holds_the_partial_states(dtype, Nq, d):
    """The workspace layout documented in fa.h: m [S][rows], l [S][rows], acc
    [S][rows][d] at the next 256-byte boundary.  Each range's state must match
    the oracle's partial_state of that key range (compared through quantities
    that do not depend on the reference: m*scale + ln l and acc / l).  One
    query row in bf16 runs the decoding pass."""
    B, H, Nk, S = 1, 2, 1000, 4
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=2400, dtype=dtype)
    scale = inputs.default_scale(d)
    nbytes = fa.fa_splitkv_workspace_bytes(B, H, Nq, d, S)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN-filled
    run_split(q, k, v, scale, num_splits=S, workspace=ws)
    rows = B * H * Nq
    wsf = ws.view(torch.float32).cpu().numpy()
    m, l = wsf[:S * rows].reshape(S, rows), wsf[S * rows:2 * S * rows].reshape(S, rows)
    off = ((2 * S * rows * 4 + 255) // 256) * 256 // 4
    acc = wsf[off:off + S * rows * d].reshape(S, rows, d)
    qn, kn, vn = (to_np32(x).astype(np.float64) for x in (q, k, v))
    tiles = (Nk + 63) // 64
    for r in range(rows):
        bh, i = divmod(r, Nq)
        s = scale * (kn.reshape(B * H, Nk, d)[bh] @ qn.reshape(B * H, Nq, d)[bh, i])
        for part in range(S):
            lo = min(Nk, part * tiles // S * 64)
            hi = min(Nk, (part + 1) * tiles // S * 64)
            ref = partial_state(s[lo:hi], vn.reshape(B * H, Nk, d)[bh, lo:hi])
            assert abs(m[part, r] * scale - ref["m"]) < 1e-5
            lse_p = m[part, r] * scale + math.log(l[part, r])
            assert abs(lse_p - (ref["m"] + math.log(ref["l"]))) < 1e-5
            assert np.max(np.abs(acc[part, r] / l[part, r] - ref["o_tilde"] / ref["l"])) < 1e-5


def test_splitkv_reuses_a_workspace():
    """Two calls in a row on one workspace, the second smaller: its contents
    on entry do not matter."""
    d = 128
    scale = inputs.default_scale(d)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(2, 4, 64, d, 8), dtype=torch.uint8, device=DEV)
    for (B, H, Nq, Nk, S) in ((2, 4, 64, 3000, 8), (1, 3, 7, 500, 5)):
        q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=2500 + Nk, dtype="bf16")
        o, lse = run_split(q, k, v, scale, num_splits=S, workspace=ws)
        o_ref, lse_ref = run_oracle(q, k, v, scale)
        compare(o, lse, o_ref, lse_ref, "bf16", what="reuse Nk=%d" % Nk)


def test_splitkv_matches_the_plain_pass():
    """Split and plain pass on the same causal inputs: both within the bar of
    the oracle, and within the bf16 bar of each other."""
    q, k, v = inputs.gaussian_qkv(1, 2, 2048, 2048, 128, seed=2600, dtype="bf16")
    scale = inputs.default_scale(128)
    o_s, lse_s = run_split(q, k, v, scale, causal=True, num_splits=4)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o_p, lse_p = fa.attention(qd, kd, vd, scale=scale, causal=True)
    torch.cuda.synchronize()
    o_p = o_p.float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o_s - o_p)) <= 2e-2
    assert np.max(np.abs(lse_s - lse_p.cpu().numpy())) <= 1e-3
    rows = np.arange(0, 2 * 2048, 37)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=True, rows=rows)
    compare(o_s.reshape(-1, 128)[rows], lse_s.reshape(-1)[rows], o_ref, lse_ref, "bf16",
            what="split vs oracle")


# ---------------------------------------------------------------------------
# fa_merge_states
# ---------------------------------------------------------------------------
def _random_states(n_parts, rows, d, seed):
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal((n_parts, rows)) * 30).astype(np.float32)
    m[rng.random((n_parts, rows)) < 0.2] = -np.inf          # parts without a visible key
    m[:, 7] = -np.inf                                        # a row with none at all
    l = (1.0 + rng.random((n_parts, rows)) * 50).astype(np.float32)
    acc = (rng.standard_normal((n_parts, rows, d)) * l[..., None]).astype(np.float32)
    l[np.isneginf(m)] = 0.0
    acc[np.isneginf(m)] = 0.0
    return m, l, acc


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_merge_states_matches_the_oracle_merge(d, out):
    n_parts, rows, scale = 5, 301, 0.37
    m, l, acc = _random_states(n_parts, rows, d, seed=2700 + d)
    o, lse = fa.merge_states(*(torch.from_numpy(x).to(DEV) for x in (m, l, acc)), scale,
                             out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy()
    o_ref = np.zeros((rows, d))
    lse_ref = np.zeros(rows)
    for r in range(rows):
        st = [{"m": float(m[i, r]) * scale, "l": float(l[i, r]),
               "o_tilde": acc[i, r].astype(np.float64)} for i in range(n_parts)]
        res = merge_states(st)
        o_ref[r], lse_ref[r] = res["o"], res["lse"]
    compare(o, lse, o_ref, lse_ref, out, what="merge d=%d %s" % (d, out))


def test_merge_of_oracle_partial_states_gives_attention():
    """The exchange step end to end: partial states of consecutive key ranges
    from the oracle, merged on the GPU, equal the three-pass result over all
    keys."""
    B, H, Nq, Nk, d = 1, 2, 9, 777, 128
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed=2800, dtype="f32")
    scale = inputs.default_scale(d)
    qn, kn, vn = (to_np32(x).astype(np.float64).reshape(B * H, -1, d) for x in (q, k, v))
    cuts = [0, 100, 101, 400, 777]
    P, rows = len(cuts) - 1, B * H * Nq
    m = np.zeros((P, rows), np.float32)
    l = np.zeros((P, rows), np.float32)
    acc = np.zeros((P, rows, d), np.float32)
    for r in range(rows):
        bh, i = divmod(r, Nq)
        s = scale * (kn[bh] @ qn[bh, i])
        for p_, (lo, hi) in enumerate(zip(cuts, cuts[1:])):
            st = partial_state(s[lo:hi], vn[bh, lo:hi])
            # the library states the reference in raw score units
            m[p_, r], l[p_, r], acc[p_, r] = st["m"] / scale, st["l"], st["o_tilde"]
    o, lse = fa.merge_states(*(torch.from_numpy(x).to(DEV) for x in (m, l, acc)), scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = run_oracle(q, k, v, scale)
    compare(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), o_ref.reshape(rows, d),
            lse_ref.reshape(rows), "f32", what="merged oracle partials")
