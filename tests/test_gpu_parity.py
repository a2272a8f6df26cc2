"""GPU parity: the HIP path (through the C ABI binding) against the fp64 oracle
on the same seeded inputs, element by element.

Workloads (online_softmax_fa_amd.inputs): the small fp32 case and the pages'
toy rows; the adversarial exact-score heads with every mask case, both
dtypes, every tile size and both traversal orders; the mid-size causal bf16
case and the headline causal bf16 case on every row, and the long-context
case on one whole head plus sampled rows (at the launch configuration the
bench times); and edge shapes (ragged tails, one key, one query, fully
masked rows and batches).
"""

import math

import numpy as np
import pytest
import torch

from online_softmax_fa_amd import inputs
from _parity import compare, run_gpu, run_oracle, sample_rows, say, to_np32

pytestmark = pytest.mark.gpu

BLOCKS = (16, 32, 64, 128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_fa_amd as fa
    fa.load_library()
    props = torch.cuda.get_device_properties(0)
    say("device: %s %s" % (props.name, getattr(props, "gcnArchName", "")))


# ---------------------------------------------------------------------------
def test_small_fp32():
    w = inputs.workload("small")
    say("small fp32 B=1 H=1 N=256 d=64")
    o, lse = run_gpu(w["q"], w["k"], w["v"], w["scale"])
    o_ref, lse_ref = run_oracle(w["q"], w["k"], w["v"], w["scale"])
    compare(o, lse, o_ref, lse_ref, "f32", what="small")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_all_tiles_agree(dtype):
    w = inputs.workload("small", dtype=dtype)
    o_ref, lse_ref = run_oracle(w["q"], w["k"], w["v"], w["scale"])
    outs = []
    for bn in BLOCKS:
        for rev in (False, True):
            say("small %s block_n=%d reverse=%d" % (dtype, bn, rev))
            o, lse = run_gpu(w["q"], w["k"], w["v"], w["scale"], block_n=bn, reverse_kv=rev)
            compare(o, lse, o_ref, lse_ref, dtype, what="bn%d rev%d" % (bn, rev))
            outs.append(o)
    bar = 1e-5 if dtype == "f32" else 2e-2
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= bar


def _toy_tensors(scores, values, d=64):
    """A precomputed score row fed through the library: one query q = e0 and
    keys k_j = s_j e0 with scale 1, so every score is exact; values occupy the
    first columns."""
    n = len(scores)
    q = torch.zeros(1, 1, 1, d)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, n, d)
    k[0, 0, :, 0] = torch.tensor(scores, dtype=torch.float32)
    v = torch.zeros(1, 1, n, d)
    vals = torch.tensor(values, dtype=torch.float32).reshape(n, -1)
    v[0, 0, :, :vals.shape[1]] = vals
    return q, k, v


@pytest.mark.parametrize("bn", BLOCKS)
def test_pages_toy_rows(bn):
    """'2.2b', 'The Softmax Formula' (S=[2,4,1,3] -> [0.087, 0.644, 0.032,
    0.237]); 'The math of FlashAttention', 'A fully worked numeric example'
    (s=[1,3,2,5], v=[10,20,30,40] -> 36.88)."""
    q, k, v = _toy_tensors([2, 4, 1, 3], np.eye(4))
    o, lse = run_gpu(q, k, v, 1.0, block_n=bn)
    assert np.max(np.abs(o[0, 0, 0, :4] - np.array([0.087, 0.644, 0.032, 0.237]))) <= 5e-4
    assert np.all(o[0, 0, 0, 4:] == 0.0)
    assert abs(math.exp(lse[0, 0, 0]) - 84.80) <= 0.02
    o_ref, lse_ref = run_oracle(q, k, v, 1.0)
    compare(o, lse, o_ref, lse_ref, "f32", what="toy1 bn%d" % bn)

    q, k, v = _toy_tensors([1, 3, 2, 5], [[10], [20], [30], [40]])
    o, lse = run_gpu(q, k, v, 1.0, block_n=bn)
    assert abs(o[0, 0, 0, 0] - 36.88) <= 5e-3
    o_ref, lse_ref = run_oracle(q, k, v, 1.0)
    compare(o, lse, o_ref, lse_ref, "f32", what="toy2 bn%d" % bn)    # the plain 1e-5 bar

    q, k, v = _toy_tensors([1, 2, 5, 3], [[1, 0], [0, 1], [2, 0], [0, 2]])
    o, lse = run_gpu(q, k, v, 1.0, block_n=bn)
    assert np.max(np.abs(o[0, 0, 0, :2] - np.array([1.677, 0.266]))) <= 5e-4


# ---------------------------------------------------------------------------
# Adversarial heads: exact scores, max in the last / first tile, max jumps that
# underflow alpha, maxima straddling ln(FLT_MAX), key-padding masks, fully
# masked rows; every tile size and both traversal orders.
# ---------------------------------------------------------------------------
ADV_CASES = list(inputs.adversarial_cases().keys())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ADV_CASES)
def test_adversarial(dtype, case):
    q, k, v = inputs.adversarial(dtype=dtype)
    mask, causal = inputs.adversarial_cases()[case]
    say("adversarial %s %s causal=%d" % (dtype, case, causal))
    o_ref, lse_ref = run_oracle(q, k, v, inputs.ADV_SCALE, causal=causal, mask=mask)
    outs = []
    for bn in BLOCKS:
        for rev in (False, True):
            o, lse = run_gpu(q, k, v, inputs.ADV_SCALE, causal=causal, mask=mask, block_n=bn,
                             reverse_kv=rev)
            compare(o, lse, o_ref, lse_ref, dtype, what="%s bn%d rev%d" % (case, bn, rev))
            outs.append(o)
    bar = 1e-5 if dtype == "f32" else 2e-2
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= bar


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_maxima(dtype, causal):
    """Row maxima that keep rising across the keys: the running maximum moves
    by small steps on most tiles (head 0), by large steps on every tile
    (head 2), slowly (head 3), or never after the first tile (head 1)."""
    q, k, v = inputs.adversarial_ramps(dtype=dtype)
    say("rising maxima %s causal=%d" % (dtype, causal))
    o_ref, lse_ref = run_oracle(q, k, v, inputs.ADV_SCALE, causal=causal)
    for bn in BLOCKS:
        for rev in (False, True):
            o, lse = run_gpu(q, k, v, inputs.ADV_SCALE, causal=causal, block_n=bn,
                             reverse_kv=rev)
            compare(o, lse, o_ref, lse_ref, dtype, what="ramps bn%d rev%d" % (bn, rev))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adversarial_random_scaled(dtype):
    """Gaussian Q, K scaled so |scores| reach about 80.  bf16 is held to the
    bf16 bar.  For fp32 the scores themselves carry fp32 rounding before any
    softmax arithmetic: with |delta s_j| <= d * 2^-24 * scale * sum_c |q_c k_jc|
    (a bound on any fp32 dot-product order), the output moves by at most
    2 * max_j |delta s_j| * max |v| (first order), so that bound (plus 1e-5) is
    the fp32 bar for this case."""
    q, k, v = inputs.adversarial_random(dtype=dtype)
    o_ref, lse_ref = run_oracle(q, k, v, inputs.ADV_SCALE)
    if dtype == "f32":
        qa, ka = np.abs(to_np32(q)).astype(np.float64), np.abs(to_np32(k)).astype(np.float64)
        worst = (qa @ np.swapaxes(ka, -1, -2)).max() * inputs.ADV_SCALE
        ds = 64 * 2.0 ** -24 * worst
        bar = 1e-5 + 2 * ds * np.abs(to_np32(v)).max()
        lse_bar = max(1e-3, 2 * ds)
    else:
        bar, lse_bar = None, 1e-3
    say("adversarial random-scaled %s: fp32 bar %s" % (dtype, bar))
    s_max = float(np.abs(np.asarray(lse_ref)).max())
    assert s_max > 40.0            # the case really reaches large logits
    for bn in (32, 64, 128):
        o, lse = run_gpu(q, k, v, inputs.ADV_SCALE, block_n=bn)
        compare(o, lse, o_ref, lse_ref, dtype, max_abs=bar, lse_tol=lse_bar, what="bn%d" % bn)


# ---------------------------------------------------------------------------
# Edge shapes: ragged tails on both sides, one key, one query, d = 128 in fp32
# ---------------------------------------------------------------------------
EDGE = [
    # (B, H, Nq, Nk, d, causal, masked)
    (1, 1, 1, 1, 64, False, False),
    (1, 2, 1, 4, 64, False, False),
    (2, 3, 33, 33, 64, True, False),
    (1, 2, 100, 37, 128, False, True),
    (1, 2, 37, 100, 128, True, True),
    (2, 1, 257, 300, 64, False, True),
    (1, 1, 129, 1, 128, False, False),
    (1, 3, 300, 257, 128, True, False),
    (3, 2, 64, 64, 64, True, True),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE, ids=["x".join(map(str, s[:5])) + ("c" if s[5] else "")
                                             + ("m" if s[6] else "") for s in EDGE])
def test_edge_shapes(dtype, shape):
    B, H, Nq, Nk, d, causal, masked = shape
    seed = 5000 + Nq * 7 + Nk
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed, 1.0, dtype)
    mask = None
    if masked:
        mask = inputs.bernoulli_mask(B, Nk, 0.3, seed + 1)
        mask[0, : min(5, Nk)] = 0
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask)
    for bn in (16, 32, 64, 128):
        say("edge %s %s bn=%d" % (dtype, shape, bn))
        o, lse = run_gpu(q, k, v, scale, causal=causal, mask=mask, block_n=bn)
        compare(o, lse, o_ref, lse_ref, dtype, what="bn%d" % bn)


# ---------------------------------------------------------------------------
# 256-row workgroups (8 waves): bf16, d = 128, 64-key tiles and enough
# workgroups -- ragged query and key tails, key-padding masks with fully
# masked rows, the causal diagonal, both traversal orders
# ---------------------------------------------------------------------------
WIDE = [
    # (B, H, Nq, Nk, causal, masked): 2*64*2 = 256 and 4*256*2 = 2048 workgroups
    (2, 64, 300, 300, False, True),
    (4, 256, 257, 257, True, False),
]


@pytest.mark.parametrize("shape", WIDE, ids=["%dx%dx%dx%d%s%s" % (s[:4] + ("c" if s[4] else "",
                                                                         "m" if s[5] else ""))
                                             for s in WIDE])
def test_256_row_workgroups(shape):
    import online_softmax_fa_amd as fa
    B, H, Nq, Nk, causal, masked = shape
    d = 128
    assert fa.fa_query_tile_rows(fa.FA_DTYPE_BF16, B, H, Nq, d, 64, causal) == 256
    seed = 5600 + H
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nk, d, seed, 1.0, "bf16")
    mask = None
    if masked:
        mask = inputs.bernoulli_mask(B, Nk, 0.3, seed + 1)
        mask[1, :] = 0                      # batch 1: every row fully masked
    scale = inputs.default_scale(d)
    heads = [(0, 0), (0, H - 1), (B - 1, H // 2), (B - 1, H - 1)]
    rows = sample_rows(B, H, Nq, heads, 96, seed + 2)
    rows = np.unique(np.concatenate([rows, np.arange(Nq) + (H - 1) * Nq]))   # head (0, H-1) in full
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask, rows=rows)
    outs = []
    for rev in (False, True):
        say("256-row workgroups %s reverse=%d" % (shape, rev))
        o, lse = run_gpu(q, k, v, scale, causal=causal, mask=mask, reverse_kv=rev)
        compare(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, "bf16",
                what="wide rev%d" % rev)
        assert np.all(np.isfinite(o))
        outs.append((o, lse))
    if masked:
        o, lse = outs[0]
        assert np.all(o.reshape(B, H, Nq, d)[1] == 0.0) and np.all(np.isneginf(lse[1]))


# ---------------------------------------------------------------------------
# Paired causal query tiles: when the pairs (t, n_qt - 1 - t) of a causal
# launch fill whole rounds of the device's workgroup slots (256 CUs: one
# 8-wave workgroup or three d = 64 workgroups per CU), each workgroup takes
# both tiles of a pair one after the other.  An odd n_qt leaves the middle
# tile alone.
# ---------------------------------------------------------------------------
PAIRED = [
    # (B, H, Nq, d, masked): 8 waves, n_qt = 31 (ragged, odd), 2*16*16 = 512 pairs;
    # unmasked, the second item's first key tile is fetched during the first
    # item's last tile whenever the first item has an even tile count
    (2, 16, 7700, 128, False),
    (2, 16, 7700, 128, True),
    # 4 waves of d = 64, n_qt = 32, 48*16 = 768 pairs
    (1, 48, 4096, 64, False),
]


@pytest.mark.parametrize("shape", PAIRED, ids=["%dx%dx%dx%d%s" % (s[:4] + ("m" if s[4] else "",))
                                              for s in PAIRED])
def test_paired_causal_tiles(shape):
    B, H, Nq, d, masked = shape
    seed = 5900 + H
    q, k, v = inputs.gaussian_qkv(B, H, Nq, Nq, d, seed, 1.0, "bf16")
    mask = None
    if masked:
        lens = inputs.kv_lengths(B, Nq, seed + 1)
        mask = inputs.prefix_mask(lens, Nq)
    scale = inputs.default_scale(d)
    heads = [(0, 0), (B - 1, H - 1), (B - 1, H // 2)]
    rows = sample_rows(B, H, Nq, heads, 256, seed + 2)
    rows = np.unique(np.concatenate([rows, np.arange(Nq) + (H // 3) * Nq]))   # one head in full
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=True, mask=mask, rows=rows)
    for rev in (False, True):
        say("paired causal tiles %s reverse=%d" % (shape, rev))
        o, lse = run_gpu(q, k, v, scale, causal=True, mask=mask, reverse_kv=rev)
        compare(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, "bf16",
                what="paired rev%d" % rev)
        assert np.all(np.isfinite(o))


def _span_mask(N):
    """Key-padding masks whose visible keys sit inside the key range, so that
    whole key tiles before and after them are skipped: batch 0 sees keys
    150..529 only, batch 1 the single key 333, batch 2 the last 3 keys.  With
    N odd the mask rows start at unaligned byte offsets."""
    m = torch.zeros(3, N, dtype=torch.uint8)
    m[0, 150:530] = 1
    m[1, 333] = 1
    m[2, N - 3:] = 1
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mask_spans(dtype, d, causal):
    """Visible keys only in the middle, at one key, or at the end of the key
    range, at every tile size and both orders, and through the split-key
    path: the tiles outside the span are never visited, and rows that see no
    key get o = 0 and lse = -inf exactly."""
    import online_softmax_fa_amd as fa
    B, H, N = 3, 2, 701
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, 5800 + d + causal, 1.0, dtype)
    mask = _span_mask(N)
    scale = inputs.default_scale(d)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask)
    for bn in BLOCKS:
        for rev in (False, True):
            say("mask spans %s d=%d causal=%d bn=%d reverse=%d" % (dtype, d, causal, bn, rev))
            o, lse = run_gpu(q, k, v, scale, causal=causal, mask=mask, block_n=bn, reverse_kv=rev)
            compare(o, lse, o_ref, lse_ref, dtype, what="spans bn%d rev%d" % (bn, rev))
            if causal:   # rows before the first visible key see nothing
                assert np.all(o[0, :, :150] == 0) and np.all(np.isneginf(lse[0, :, :150]))
                assert np.all(o[2, :, :N - 3] == 0) and np.all(np.isneginf(lse[2, :, :N - 3]))
    dev = torch.device("cuda:0")
    for ns in (2, 5):
        say("mask spans split-key %s d=%d causal=%d splits=%d" % (dtype, d, causal, ns))
        o, lse = fa.attention_splitkv(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal,
                                      kv_len_mask=mask.to(dev), num_splits=ns)
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), o_ref, lse_ref,
                dtype, what="spans split %d" % ns)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nk", [1, 63, 5000])
@pytest.mark.parametrize("causal", [False, True])
def test_single_query_row(d, Nk, causal):
    """fa_fwd with one query row per (batch, head) in bf16 and the library's
    tile (the decoding pass, all keys in one workgroup), with per-batch key
    lengths and a batch whose keys are all masked."""
    B, H = 3, 2
    q, k, v = inputs.gaussian_qkv(B, H, 1, Nk, d, 5900 + Nk + d, 1.0, "bf16")
    mask = inputs.prefix_mask(inputs.kv_lengths(B, Nk, 5950 + Nk, lo=1), Nk)
    mask[1] = 0
    scale = inputs.default_scale(d)
    say("single query row d=%d Nk=%d causal=%d" % (d, Nk, causal))
    o, lse = run_gpu(q, k, v, scale, causal=causal, mask=mask)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal=causal, mask=mask)
    compare(o, lse, o_ref, lse_ref, "bf16", what="single row")
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_fully_masked_batch_and_rows():
    B, H, N, d = 3, 2, 96, 64
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, 77, 1.0, "bf16")
    mask = torch.ones(B, N, dtype=torch.uint8)
    mask[0] = 0                 # batch 0: no key at all
    mask[1, :50] = 0            # batch 1 causal: rows 0..49 see nothing
    o, lse = run_gpu(q, k, v, 0.125, causal=True, mask=mask)
    o_ref, lse_ref = run_oracle(q, k, v, 0.125, causal=True, mask=mask)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(o[1, :, :50] == 0) and np.all(np.isneginf(lse[1, :, :50]))
    compare(o, lse, o_ref, lse_ref, "bf16", what="masked batch")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_weights_sum_to_one_and_causal_row0(dtype):
    """A constant value column comes back unchanged (the weights sum to 1);
    causal row 0 sees only key 0, so o = v_0 exactly."""
    B, H, N, d = 2, 4, 200, 128
    q, k, v = inputs.gaussian_qkv(B, H, N, N, d, 88, 2.0, dtype)
    v[..., 5] = 1.0
    o, lse = run_gpu(q, k, v, inputs.default_scale(d), causal=True)
    # bf16: the weights are rounded to bf16 for the product while l sums them
    # in fp32, and o is rounded to bf16: within one bf16 step below 1.  fp32:
    # l and the product sum the same n weights in two different fp32 orders,
    # each within (n - 1) * 2^-24 relative, so n * 2^-23 bounds the difference.
    tol = 2.0 ** -8 if dtype == "bf16" else N * 2.0 ** -23
    assert np.max(np.abs(o[..., 5] - 1.0)) <= tol
    v0 = to_np32(v)[:, :, 0, :].astype(np.float64)
    assert np.array_equal(o[:, :, 0, :], v0)


# ---------------------------------------------------------------------------
# Larger workloads
# ---------------------------------------------------------------------------
def test_mid_causal_bf16_and_determinism():
    w = inputs.workload("mid")
    say("mid bf16 causal B=4 H=16 N=2048 d=64")
    q, k, v = w["q"], w["k"], w["v"]
    o, lse = run_gpu(q, k, v, w["scale"], causal=True)
    o_ref, lse_ref = run_oracle(q, k, v, w["scale"], causal=True)     # every row
    compare(o, lse, o_ref, lse_ref, "bf16", what="mid")
    o2, lse2 = run_gpu(q, k, v, w["scale"], causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "run-to-run difference"


def test_headline_every_row():
    """The headline workload at its full size, in the launch configuration the
    bench times, against the oracle on all 524288 rows (about 1.1e12 fp64
    FLOP: seconds on a many-core host)."""
    w = inputs.workload("headline")
    say("headline bf16 causal B=2 H=32 N=8192 d=128 (every row)")
    q, k, v = w["q"], w["k"], w["v"]
    o, lse = run_gpu(q, k, v, w["scale"], causal=True)
    o_ref, lse_ref = run_oracle(q, k, v, w["scale"], causal=True)
    compare(o, lse, o_ref, lse_ref, "bf16", what="headline")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("masked", [False, True])
def test_long_sampled(masked):
    w = inputs.workload("long")
    q, k, v = w["q"], w["k"], w["v"]
    mask = None
    if masked:
        lens = inputs.kv_lengths(1, 32768, 2005)
        mask = inputs.prefix_mask(lens, 32768)
        say("long bf16 B=1 H=8 N=32768 d=128, kv length %d" % int(lens[0]))
    else:
        say("long bf16 B=1 H=8 N=32768 d=128")
    o, lse = run_gpu(q, k, v, w["scale"], mask=mask)
    # head 3 on every row (5.5e11 fp64 FLOP), sampled rows of heads 0 and 5
    rows = sample_rows(1, 8, 32768, [(0, 0), (0, 5)], 64, 13)
    rows = np.unique(np.concatenate([rows, np.arange(32768) + 3 * 32768]))
    o_ref, lse_ref = run_oracle(q, k, v, w["scale"], mask=mask, rows=rows)
    compare(o.reshape(-1, 128)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, "bf16",
            what="long masked=%d" % masked)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
