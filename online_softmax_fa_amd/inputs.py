"""Seeded synthetic inputs for the attention forward pass.

This module only draws and arranges numbers: it holds none of the attention
arithmetic, so both the HIP path's tests/bench and the CPU oracle can take
their inputs from it without sharing any computation.

Every tensor is drawn on the CPU in float32 from ``torch.Generator`` with a
fixed seed, then rounded to bfloat16 (round-to-nearest-even) when the case is
bf16.  The oracle receives the very same values widened back to float32,
which is exact.

Workloads (shapes, value distributions and masks):

  small      B=1 H=1 N=256 d=64 fp32, Q/K/V ~ N(0,1), scale 1/8, no mask
  adv        B=1 H=4 N=1024 d=64, fp32 and bf16, scores built to be exact
             (see ``adversarial``), key-padding masks with 10-50% of keys
             masked, fully masked rows
  mid        B=4 H=16 N=2048 d=64 bf16 causal, Q/K/V ~ N(0,1)
  headline   B=2 H=32 N=8192 d=128 bf16 causal, Q/K/V ~ N(0,1)
  long       B=1 H=8 N=32768 d=128 bf16 non-causal, Q/K/V ~ N(0, 0.5^2),
             plus per-batch key lengths uniform in [N/2, N] as a prefix mask
  decode     B=8 H=8 N_q=1 N_k=32768 d=128 bf16 non-causal, N(0, 0.5^2): one
             new query per sequence over the long-context geometry
  softmax    8192 score rows of 8192 fp32 entries ~ N(0, 1) (one head of the
             headline's score matrix), for the standalone row softmax
"""

import math

import torch

WORKLOADS = {
    "small": dict(B=1, H=1, N=256, d=64, dtype="f32", causal=False, std=1.0, seed=1001),
    "adv": dict(B=1, H=4, N=1024, d=64, dtype="f32", causal=False, std=1.0, seed=1002),
    "mid": dict(B=4, H=16, N=2048, d=64, dtype="bf16", causal=True, std=1.0, seed=1003),
    "headline": dict(B=2, H=32, N=8192, d=128, dtype="bf16", causal=True, std=1.0, seed=1004),
    "long": dict(B=1, H=8, N=32768, d=128, dtype="bf16", causal=False, std=0.5, seed=1005),
    # one new query per sequence over the long-context cache geometry (8 heads,
    # 32768 keys, d = 128, N(0, 0.5^2)), 8 sequences: the split-key path
    "decode": dict(B=8, H=8, N=32768, Nq=1, d=128, dtype="bf16", causal=False, std=0.5,
                   seed=1006),
}

# Score rows for the standalone row softmax: one head's full score matrix of
# the headline shape (8192 x 8192), whose entries q.k / sqrt(d) are N(0, 1)
# for N(0, 1) queries and keys.
ROW_WORKLOADS = {
    "softmax": dict(rows=8192, n=8192, dtype="f32", std=1.0, seed=1007),
}


def row_workload(name):
    w = dict(ROW_WORKLOADS[name])
    w["s"] = gaussian((w["rows"], w["n"]), w["seed"], w["std"], w["dtype"])
    return w

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def default_scale(d):
    """1/sqrt(d) rounded to float32: the value handed to the library."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def gaussian(shape, seed, std=1.0, dtype="f32"):
    """i.i.d. N(0, std^2) in float32, then cast to `dtype` ("f32" or "bf16")."""
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPE[dtype])


def gaussian_qkv(B, H, Nq, Nk, d, seed, std=1.0, dtype="f32"):
    q = gaussian((B, H, Nq, d), seed * 3 + 0, std, dtype)
    k = gaussian((B, H, Nk, d), seed * 3 + 1, std, dtype)
    v = gaussian((B, H, Nk, d), seed * 3 + 2, std, dtype)
    return q, k, v


def bernoulli_mask(B, Nk, masked_fraction, seed):
    """uint8 [B, Nk]: each key masked (0) independently with the given probability."""
    u = torch.rand(B, Nk, generator=_gen(seed))
    return (u >= masked_fraction).to(torch.uint8)


def kv_lengths(B, Nk, seed, lo=None, hi=None):
    """Per-batch key lengths drawn uniformly from [lo, hi] (default [Nk/2, Nk])."""
    lo = Nk // 2 if lo is None else lo
    hi = Nk if hi is None else hi
    return torch.randint(lo, hi + 1, (B,), generator=_gen(seed))


def prefix_mask(lengths, Nk):
    """uint8 [B, Nk]: key j of batch b visible iff j < lengths[b]."""
    j = torch.arange(Nk).unsqueeze(0)
    return (j < lengths.view(-1, 1)).to(torch.uint8)


def workload(name, dtype=None, seed=None):
    """Q, K, V (and the run parameters) of one named workload without masks."""
    w = dict(WORKLOADS[name])
    if dtype is not None:
        w["dtype"] = dtype
    if seed is not None:
        w["seed"] = seed
    nq = w.get("Nq", w["N"])
    q, k, v = gaussian_qkv(w["B"], w["H"], nq, w["N"], w["d"], w["seed"], w["std"], w["dtype"])
    return dict(q=q, k=k, v=v, scale=default_scale(w["d"]), causal=w["causal"], mask=None,
                dtype=w["dtype"], std=w["std"], Nq=nq, **{k2: w[k2] for k2 in ("B", "H", "N", "d")})


# ---------------------------------------------------------------------------
# Adversarial rows with exactly representable scores.
#
# q_i = [8, a_i1 .. a_i63] and k_j = [t_j, b_j1 .. b_j63] with a, b in
# {-1, 0, 1} and integer offsets t_j; with scale 1/8 the score is
# s_ij = t_j + n_ij / 8 for an integer n_ij in [-63, 63].  Every product and
# partial sum is an integer below 2^24, so fp32 and bf16 inputs give the same
# exact scores on any hardware.  Per head:
#   head 0: t_j = 78 on the last 16 keys, uniform integers in [-80, 60]
#           elsewhere: every row's maximum sits in the last tile
#   head 1: head 0 with the key order reversed: the maximum sits in the first
#   head 2: last 16 keys 78, elsewhere [-80, -60]: the maximum jumps by > 130,
#           so the rescale factor underflows to 0 in fp32
#   head 3: offsets [-80, 60] with 16 spike keys at t = 86 spread over the
#           row, so maxima straddle ln(FLT_MAX) = 88.72
# ---------------------------------------------------------------------------
ADV_SCALE = 0.125


def adversarial(seed=1002, N=1024, dtype="f32"):
    d = 64
    H = 4
    g = _gen(seed)
    q = torch.zeros(1, H, N, d)
    k = torch.zeros(1, H, N, d)
    q[..., 0] = 8.0
    q[..., 1:] = torch.randint(-1, 2, (1, H, N, d - 1), generator=g).float()
    k[..., 1:] = torch.randint(-1, 2, (1, H, N, d - 1), generator=g).float()
    t0 = torch.randint(-80, 61, (N,), generator=g).float()
    t0[N - 16:] = 78.0
    t2 = torch.randint(-80, -59, (N,), generator=g).float()
    t2[N - 16:] = 78.0
    t3 = torch.randint(-80, 61, (N,), generator=g).float()
    spikes = torch.randperm(N, generator=g)[:16]
    t3[spikes] = 86.0
    k[0, 0, :, 0] = t0
    k[0, 2, :, 0] = t2
    k[0, 3, :, 0] = t3
    v = torch.randn(1, H, N, d, generator=g)
    # head 1: the keys (and their values) of head 0 in reverse order
    k[0, 1] = torch.flip(k[0, 0], dims=[0])
    v[0, 1] = torch.flip(v[0, 0], dims=[0])
    dt = TORCH_DTYPE[dtype]
    return q.to(dt), k.to(dt), v.to(dt)


def adversarial_random(seed=1012, N=1024, dtype="f32", target=80.0):
    """Gaussian Q, K scaled so that the largest |score| is about `target`."""
    d = 64
    g = _gen(seed)
    q = torch.randn(1, 4, N, d, generator=g)
    k = torch.randn(1, 4, N, d, generator=g)
    v = torch.randn(1, 4, N, d, generator=g)
    # raw scores with scale 1/8 have standard deviation 1; the max of 4M
    # such values is about 5, so each side is scaled by sqrt(target / 5)
    gamma = math.sqrt(target / 5.0)
    dt = TORCH_DTYPE[dtype]
    return (q * gamma).to(dt), (k * gamma).to(dt), v.to(dt)


def adversarial_cases(N=1024, seed=1002):
    """Named (mask, causal) combinations run on the adversarial heads.

    Masks are [1, N] uint8 shared by the four heads.
    """
    cases = {"nomask": (None, False)}
    for i, r in enumerate((0.1, 0.3, 0.5)):
        cases["bern%02d" % int(r * 100)] = (bernoulli_mask(1, N, r, seed + 100 + i), False)
    m = torch.ones(1, N, dtype=torch.uint8)
    m[0, N - 16:] = 0      # the keys holding head 0's maximum
    cases["mask_max_keys"] = (m, False)
    m = torch.ones(1, N, dtype=torch.uint8)
    m[0, :40] = 0          # rows 0..39 have no visible key under causality
    cases["causal_prefix_masked"] = (m, True)
    cases["causal"] = (None, True)
    cases["all_masked"] = (torch.zeros(1, N, dtype=torch.uint8), False)
    return cases


def adversarial_ramps(seed=1022, N=1024, dtype="f32"):
    """Exact scores whose row maximum keeps rising across the keys.

    Same construction as ``adversarial`` (scale 1/8, s = t_j + n/8), with
    integer offsets t_j that ramp with the key index:
      head 0: t_j = j // 16 - 32      (+4 per 64 keys: moderate growth)
      head 1: head 0 reversed         (the maximum comes first)
      head 2: t_j = j // 4 - 128      (+16 per 64 keys: the maximum jumps
                                       every tile)
      head 3: t_j = j // 64 - 8       (+1 per 64 keys: slow drift)
    """
    d, H = 64, 4
    g = _gen(seed)
    q = torch.zeros(1, H, N, d)
    k = torch.zeros(1, H, N, d)
    q[..., 0] = 8.0
    q[..., 1:] = torch.randint(-1, 2, (1, H, N, d - 1), generator=g).float()
    k[..., 1:] = torch.randint(-1, 2, (1, H, N, d - 1), generator=g).float()
    j = torch.arange(N)
    k[0, 0, :, 0] = (j // 16 - 32).float()
    k[0, 2, :, 0] = (j // 4 - 128).float()
    k[0, 3, :, 0] = (j // 64 - 8).float()
    v = torch.randn(1, H, N, d, generator=g)
    k[0, 1] = torch.flip(k[0, 0], dims=[0])
    v[0, 1] = torch.flip(v[0, 0], dims=[0])
    dt = TORCH_DTYPE[dtype]
    return q.to(dt), k.to(dt), v.to(dt)
