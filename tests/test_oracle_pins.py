"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each check compares the oracle with something other than itself:
  - numbers the pages print in their worked examples (tests/golden), at half a
    unit of the last printed digit;
  - closed forms (one key, equal scores, constant values, causal row 0);
  - invariants the pages state (weights sum to 1, shift invariance, key
    permutation, block size and order independence);
  - brute force of the plain definition, without max subtraction, in 50-digit
    decimal arithmetic on tiny inputs;
  - the textbook special case computed by a library routine (torch fp64
    softmax followed by a matrix product);
  - for the merge of partial states: the pages' two-block example, and the
    three-pass oracle over the union of the key ranges.
"""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle.online import merge_states, online_attention_row, partial_state

# Mutation testing (tests/test_oracle_mutants.py) reruns this file against
# copies of the oracle with a planted mistake; these variables point there.
_MUTANT_LIB = os.environ.get("FA_TEST_MUTANT_ORACLE_LIB")
if _MUTANT_LIB:
    oracle._LIB = _MUTANT_LIB
    oracle._lib = None
_MUTANT_ONLINE = os.environ.get("FA_TEST_MUTANT_ONLINE_SRC")
if _MUTANT_ONLINE:
    import importlib.util
    _spec = importlib.util.spec_from_file_location("online_mutant", _MUTANT_ONLINE)
    _mod = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_mod)
    online_attention_row = _mod.online_attention_row
    partial_state = _mod.partial_state
    merge_states = _mod.merge_states

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))


def _case(section, cid):
    for c in GOLDEN[section]:
        if c["id"] == cid:
            return c
    raise KeyError(cid)


def setup_module(module):
    if not _MUTANT_LIB:
        oracle.build(force=False)


# ---------------------------------------------------------------------------
# Printed values of the pages
# ---------------------------------------------------------------------------
def test_toy_softmax_row():
    c = _case("softmax_rows", "toy1_softmax")
    p, m, l = oracle.softmax_row(c["scores"])
    assert np.max(np.abs(p - np.array(c["p"]))) <= c["p_tol"]
    assert m == c["m"]
    assert abs(l - c["l"]) <= c["l_tol"]
    o, lse = oracle.attn_from_scores(c["scores"], np.eye(4))
    # one-hot values: the output is the weight vector itself
    assert np.max(np.abs(o - p)) == 0.0
    assert abs(math.exp(lse) - c["exp_lse"]) <= c["exp_lse_tol"]
    assert abs(np.sum(p) - 1.0) < 1e-15


def test_large_scores_match_printed_exponentials():
    c = _case("softmax_rows", "large_scores")
    p, m, l = oracle.softmax_row(c["scores"])
    _, lse = oracle.attn_from_scores(c["scores"], np.ones((4, 1)))
    page_lse = math.log(sum(c["page_exps"]))
    assert abs(lse - page_lse) < 5e-3
    p_shift, _, _ = oracle.softmax_row([1, 3, 0, 2])
    assert np.max(np.abs(p - p_shift)) < 1e-15
    assert m == 102


def test_scores_beyond_fp64_exp_overflow():
    c = _case("softmax_rows", "beyond_fp64_overflow")
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float64(1000.0)))
    p, m, l = oracle.softmax_row(c["scores"])
    p_shift, _, _ = oracle.softmax_row([1, 3, 0, 2])
    assert np.all(np.isfinite(p)) and np.max(np.abs(p - p_shift)) < 1e-15
    _, lse = oracle.attn_from_scores(c["scores"], np.ones((4, 1)))
    _, lse0 = oracle.attn_from_scores([0, 2, -1, 1], np.ones((4, 1)))
    assert abs(lse - (1000.0 + lse0)) < 1e-12


@pytest.mark.parametrize("cid", ["attn_two_blocks", "attn_rescale", "scalar_values_worked"])
def test_attention_rows_final(cid):
    c = _case("attention_rows", cid)
    o, lse = oracle.attn_from_scores(c["scores"], c["values"])
    assert np.max(np.abs(o - np.array(c["o"]))) <= c["o_tol"]
    if "p" in c:
        p, _, _ = oracle.softmax_row(c["scores"])
        assert np.max(np.abs(p - np.array(c["p"]))) <= c["p_tol"]
    if "o_first_alt" in c:
        assert abs(o[0] - c["o_first_alt"]) <= c["o_first_alt_tol"]
    if "weights_exp" in c:
        s = np.array(c["scores"], dtype=float)
        p, m, l = oracle.softmax_row(s)
        assert np.max(np.abs(p * l - np.array(c["weights_exp"]))) <= c["weights_exp_tol"]
        assert abs(l - c["l"]) <= c["l_tol"]
        # o~ = o * l (the unnormalised sum the page prints)
        assert abs(o[0] * l - c["o_tilde_final"]) <= c["o_tilde_final_tol"]


# ---------------------------------------------------------------------------
# The online recurrence: the pages' block-by-block traces
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cid", ["toy1_blocks", "rescale_blocks", "q3_blocks_of_one",
                                 "q2_rescale_factor"])
def test_block_traces(cid):
    c = _case("block_traces", cid)
    r = online_attention_row(c["scores"], None, block=c["block"])
    assert len(r["trace"]) == len(c["after"])
    l_prev = 0.0
    for st, exp in zip(r["trace"], c["after"]):
        assert st["m_new"] == exp["m"]
        if "l" in exp:
            assert abs(st["l"] - exp["l"]) <= c["l_tol"]
        if "alpha" in exp:
            tol = c.get("alpha_tol", 5e-4)
            assert abs(st["alpha"] - exp["alpha"]) <= tol
        if "alpha_l_prev" in exp:
            assert abs(st["alpha"] * l_prev - exp["alpha_l_prev"]) <= c.get("l_tol", 5e-4)
        l_prev = st["l"]
    # the recurrence ends where the three-pass oracle does
    p, m, l = oracle.softmax_row(c["scores"])
    assert r["m"] == m and abs(r["l"] - l) < 1e-13


@pytest.mark.parametrize("cid", ["attn_two_blocks", "attn_rescale", "scalar_values_worked"])
def test_attention_traces(cid):
    c = _case("attention_rows", cid)
    r = online_attention_row(c["scores"], c["values"], block=c["block"])
    o_prev = None
    for st, exp in zip(r["trace"], c["after"]):
        assert st["m_new"] == exp["m"]
        if "l" in exp:
            assert abs(st["l"] - exp["l"]) <= c.get("l_trace_tol", c.get("l_tol"))
        if "o_tilde" in exp:
            assert np.max(np.abs(st["o_tilde"] - np.array(exp["o_tilde"]))) <= c["o_tilde_tol"]
        if "alpha" in exp:
            assert abs(st["alpha"] - exp["alpha"]) <= c.get("alpha_tol", 5e-4)
        if "alpha_o_prev" in exp:
            got = st["alpha"] * o_prev
            assert np.max(np.abs(got - np.array(exp["alpha_o_prev"]))) <= c["o_tilde_tol"]
        if "p" in exp:
            assert np.max(np.abs(st["p"] - np.array(exp["p"]))) <= c["p_tol"]
        o_prev = st["o_tilde"]
    o_ref, lse_ref = oracle.attn_from_scores(c["scores"], c["values"])
    assert np.max(np.abs(r["o"] - o_ref)) < 1e-13
    assert abs(r["lse"] - lse_ref) < 1e-13


def test_naive_local_max_sum_is_wrong():
    c = _case("negative_controls", "local_max_sum")
    s = np.array(c["scores"], dtype=float)
    blocks = [s[:2], s[2:]]
    naive = sum(float(np.sum(np.exp(b - b.max()))) for b in blocks)
    _, _, l = oracle.softmax_row(s)
    assert abs(l - c["correct_l"]) < 5e-4
    assert abs(naive - c["correct_l"]) > 0.1


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_single_key_gives_its_value():
    q, k, v = _rand((1, 2, 5, 8), 1), _rand((1, 2, 1, 8), 2), _rand((1, 2, 1, 8), 3)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.35)
    for h in range(2):
        for i in range(5):
            assert np.array_equal(o[0, h, i], v[0, h, 0].astype(np.float64))
            s = float(np.float32(0.35)) * float(np.dot(q[0, h, i].astype(np.float64),
                                                       k[0, h, 0].astype(np.float64)))
            assert abs(lse[0, h, i] - s) < 1e-12


def test_equal_scores_give_mean_and_log_n():
    n = 37
    q = np.zeros((1, 1, 3, 16), dtype=np.float32)
    k, v = _rand((1, 1, n, 16), 4), _rand((1, 1, n, 16), 5)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.25)
    mean = v[0, 0].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(o[0, 0] - mean)) < 1e-13
    assert np.max(np.abs(lse - math.log(n))) < 1e-13


def test_constant_values_are_returned():
    q, k = _rand((2, 3, 9, 8), 6, 3.0), _rand((2, 3, 11, 8), 7, 3.0)
    v = np.full((2, 3, 11, 8), 1.75, dtype=np.float32)
    mask = (np.random.default_rng(8).random((2, 11)) > 0.4).astype(np.uint8)
    mask[:, 0] = 1
    o, _, _ = oracle.attn_fwd(q, k, v, 0.5, causal=True, mask=mask)
    assert np.max(np.abs(o - 1.75)) < 1e-13


def test_causal_row0_is_value0():
    q, k, v = _rand((1, 2, 6, 8), 9), _rand((1, 2, 6, 8), 10), _rand((1, 2, 6, 8), 11)
    o, _, _ = oracle.attn_fwd(q, k, v, 0.3, causal=True)
    assert np.array_equal(o[0, :, 0], v[0, :, 0].astype(np.float64))


def test_fully_masked_rows():
    q, k, v = _rand((2, 2, 7, 8), 12), _rand((2, 2, 7, 8), 13), _rand((2, 2, 7, 8), 14)
    mask = np.ones((2, 7), dtype=np.uint8)
    mask[0, :] = 0          # batch 0: nothing visible
    mask[1, :3] = 0         # batch 1 causal: rows 0..2 see nothing
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.3, causal=True, mask=mask)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(o[1, :, :3] == 0.0) and np.all(np.isneginf(lse[1, :, :3]))
    assert np.all(np.isfinite(lse[1, :, 3:]))
    assert np.all(np.isfinite(o))


# ---------------------------------------------------------------------------
# Brute force of the plain definition in 50-digit decimals
# ---------------------------------------------------------------------------
def _decimal_attention(q, k, v, scale, causal, mask):
    getcontext().prec = 50
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = np.zeros((B, H, Nq, d))
    lse = np.zeros((B, H, Nq))
    sc = Decimal(float(scale))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                vis = [j for j in range(Nk)
                       if (mask is None or mask[b, j]) and (not causal or j <= i)]
                if not vis:
                    lse[b, h, i] = -math.inf
                    continue
                e = {}
                for j in vis:
                    dot = sum(Decimal(float(q[b, h, i, c])) * Decimal(float(k[b, h, j, c]))
                              for c in range(d))
                    e[j] = (sc * dot).exp()          # plain exp, no max subtraction
                den = sum(e.values())
                for c in range(d):
                    num = sum(e[j] * Decimal(float(v[b, h, j, c])) for j in vis)
                    o[b, h, i, c] = float(num / den)
                lse[b, h, i] = float(den.ln())
    return o, lse


@pytest.mark.parametrize("seed,causal,use_mask", [(20, False, False), (21, True, False),
                                                  (22, False, True), (23, True, True)])
def test_brute_force_decimal(seed, causal, use_mask):
    rng = np.random.default_rng(seed)
    B, H, Nq, Nk, d = 2, 2, 5, 7, 4
    q = (rng.standard_normal((B, H, Nq, d)) * 2).astype(np.float32)
    k = (rng.standard_normal((B, H, Nk, d)) * 2).astype(np.float32)
    v = rng.standard_normal((B, H, Nk, d)).astype(np.float32)
    mask = (rng.random((B, Nk)) > 0.3).astype(np.uint8) if use_mask else None
    if mask is not None:
        mask[0, :2] = 0
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.7, causal=causal, mask=mask)
    o_d, lse_d = _decimal_attention(q, k, v, np.float32(0.7), causal, mask)
    assert np.max(np.abs(o - o_d)) < 1e-13
    fin = np.isfinite(lse_d)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lse_d[fin])) < 1e-13


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
def test_weights_sum_to_one():
    rng = np.random.default_rng(30)
    for n in (1, 2, 17, 300):
        s = rng.standard_normal(n) * 30
        p, _, _ = oracle.softmax_row(s)
        assert abs(p.sum() - 1.0) < 1e-13 and np.all(p >= 0)


def test_shift_invariance_of_keys():
    """k_j + u for every key adds scale*(q.u) to each row's scores: o is
    unchanged and lse moves by exactly that constant ("2.2b", "The Numerical
    Stability Problem": any constant cancels).  Inputs are multiples of 1/8
    so every score, shifted or not, is exact."""
    q = np.round(_rand((1, 2, 6, 8), 31) * 8) / 8
    k = np.round(_rand((1, 2, 9, 8), 32) * 8) / 8
    v = _rand((1, 2, 9, 8), 33)
    u = np.array([0.5, -1.25, 2.0, 0.0, 3.0, -0.75, 1.0, 0.125], dtype=np.float32)
    k2 = (k + u).astype(np.float32)
    o1, l1, _ = oracle.attn_fwd(q, k, v, 0.25)
    o2, l2, _ = oracle.attn_fwd(q, k2, v, 0.25)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    shift = 0.25 * (q.astype(np.float64) @ u.astype(np.float64))
    assert np.max(np.abs((l2 - l1) - shift)) < 1e-12


def test_key_permutation_invariance():
    q, k, v = _rand((2, 2, 5, 8), 34), _rand((2, 2, 13, 8), 35), _rand((2, 2, 13, 8), 36)
    mask = (np.random.default_rng(37).random((2, 13)) > 0.3).astype(np.uint8)
    perm = np.random.default_rng(38).permutation(13)
    o1, l1, _ = oracle.attn_fwd(q, k, v, 0.4, mask=mask)
    o2, l2, _ = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.4, mask=mask[:, perm])
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


@pytest.mark.parametrize("block", [1, 2, 3, 16, 32, 64, 128, 300])
def test_block_size_and_order_do_not_change_the_result(block):
    """'Block size and traversal order never enter the result' ("The math of
    FlashAttention", "Proof of exactness")."""
    rng = np.random.default_rng(40 + block)
    n, dv = 300, 5
    s = rng.standard_normal(n) * 25
    s[-3] = 90.0                            # the max in the last block
    v = rng.standard_normal((n, dv))
    vis = rng.random(n) > 0.2
    o_ref, lse_ref = oracle.attn_from_scores(s, v.astype(np.float32), vis)
    nb = (n + block - 1) // block
    for order in (None, list(reversed(range(nb))), list(rng.permutation(nb))):
        r = online_attention_row(s, v.astype(np.float32), block=block, order=order, visible=vis)
        assert np.max(np.abs(r["o"] - o_ref)) < 1e-12
        assert abs(r["lse"] - lse_ref) < 1e-12
        ms = [t["m_new"] for t in r["trace"]]
        if order is None:
            assert all(a <= b for a, b in zip(ms, ms[1:]))      # m never decreases
        assert all(0.0 <= t["alpha"] <= 1.0 for t in r["trace"])
        assert all(np.all((t["p"] >= 0) & (t["p"] <= 1)) for t in r["trace"])


def test_masked_keys_contribute_nothing_whatever_their_score():
    """Masked keys contribute zero ("2.2b"/"The math of FlashAttention",
    "Pitfalls": mask before the block maximum).  A masked key with a huge
    score must leave the row exactly as if the key were absent."""
    rng = np.random.default_rng(70)
    s = rng.standard_normal(40) * 3
    v = rng.standard_normal((40, 3)).astype(np.float32)
    vis = np.ones(40, dtype=bool)
    vis[[5, 17, 33]] = False
    s_bad = s.copy()
    s_bad[[5, 17, 33]] = 1000.0
    o_ref, lse_ref = oracle.attn_from_scores(s[vis], v[vis])
    o1, lse1 = oracle.attn_from_scores(s_bad, v, vis)
    assert np.max(np.abs(o1 - o_ref)) < 1e-14 and abs(lse1 - lse_ref) < 1e-14
    for block in (1, 4, 16):
        r = online_attention_row(s_bad, v, block=block, visible=vis)
        assert np.max(np.abs(r["o"] - o_ref)) < 1e-13 and abs(r["lse"] - lse_ref) < 1e-13


def test_rescale_only_l_is_20x_off():
    """With the values of the first block zeroed out of the new block's
    contribution, forgetting to rescale o~ inflates o by exp(m_old - m_new)
    ("2.2b", "Check Your Understanding", question 4: m 2 -> 5 gives about
    20x).  Here the correct recurrence must match the three-pass oracle, and
    the page's factor is pinned from the old and new maxima."""
    c = _case("negative_controls", "rescale_only_l")
    s = np.array([1.0, 2.0, 5.0, 3.0])
    v = np.array([[1.0], [1.0], [0.0], [0.0]], dtype=np.float32)
    r = online_attention_row(s, v, block=2)
    o_ref, _ = oracle.attn_from_scores(s, v)
    assert abs(r["o"][0] - o_ref[0]) < 1e-13
    # the block-1 contribution after rescaling vs before: the factor the
    # page's question is about
    o_tilde_a = r["trace"][0]["o_tilde"][0]
    o_tilde_b = r["trace"][1]["o_tilde"][0]
    factor = o_tilde_a / o_tilde_b
    assert abs(factor - c["factor"]) / c["factor"] <= c["factor_tol"]


def test_online_all_masked_row():
    r = online_attention_row([1.0, 2.0, 3.0], np.ones((3, 2)), block=2, visible=[0, 0, 0])
    assert np.all(r["o"] == 0) and r["lse"] == -math.inf and r["l"] == 0.0


def test_matches_library_softmax_special_case():
    torch = pytest.importorskip("torch")
    q, k, v = _rand((2, 3, 33, 16), 50), _rand((2, 3, 41, 16), 51), _rand((2, 3, 41, 16), 52)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.25)
    qt, kt, vt = (torch.from_numpy(x).double() for x in (q, k, v))
    s = 0.25 * (qt @ kt.transpose(-1, -2).contiguous())
    ref = torch.softmax(s, dim=-1) @ vt
    assert np.max(np.abs(o - ref.numpy())) < 1e-13
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def test_row_subset_matches_full():
    q, k, v = _rand((2, 2, 20, 8), 60), _rand((2, 2, 20, 8), 61), _rand((2, 2, 20, 8), 62)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.3, causal=True)
    rows = np.array([0, 5, 19, 20, 41, 79])
    o_r, lse_r, _ = oracle.attn_fwd(q, k, v, 0.3, causal=True, rows=rows)
    assert np.array_equal(o_r, o.reshape(-1, 8)[rows])
    assert np.array_equal(lse_r, lse.reshape(-1)[rows])


# ---------------------------------------------------------------------------
# Partial states of key ranges and their merge
# ---------------------------------------------------------------------------
def test_merge_reproduces_the_pages_two_block_example():
    """The two blocks of the pages' worked example, each summarised on its own
    and then merged, give the printed state after block 1 and the printed
    final l, o~ and o, in either order ("The math of FlashAttention", "A
    fully worked numeric example")."""
    c = _case("attention_rows", "scalar_values_worked")
    s, v = np.array(c["scores"], float), np.array(c["values"], float)
    a = partial_state(s[:2], v[:2])
    b = partial_state(s[2:], v[2:])
    first = c["after"][0]
    assert a["m"] == first["m"]
    assert abs(a["l"] - first["l"]) <= c["l_trace_tol"]
    assert abs(a["o_tilde"][0] - first["o_tilde"][0]) <= c["o_tilde_tol"]
    for parts in ([a, b], [b, a]):
        r = merge_states(parts)
        assert r["m"] == c["after"][1]["m"]
        assert abs(r["l"] - c["l"]) <= c["l_tol"]
        assert abs(r["o_tilde"][0] - c["o_tilde_final"]) <= c["o_tilde_final_tol"]
        assert abs(r["o"][0] - c["o"][0]) <= c["o_tol"]


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_key_ranges_matches_the_three_pass_oracle(seed):
    """Splitting the keys of a row into consecutive ranges (some empty, some
    fully masked), summarising each and merging gives the three-pass result
    over all keys, for any order of the parts."""
    rng = np.random.default_rng(300 + seed)
    n, dv = int(rng.integers(5, 200)), 4
    s = rng.standard_normal(n) * (5 + 20 * seed)
    s[rng.integers(0, n)] += 60.0                        # one spike somewhere
    v = rng.standard_normal((n, dv)).astype(np.float32)
    vis = rng.random(n) > 0.3
    vis[: n // 5] = False                                # a fully masked leading range
    o_ref, lse_ref = oracle.attn_from_scores(s, v, vis)
    cuts = sorted(set([0, n] + list(rng.integers(0, n + 1, size=int(rng.integers(0, 6))))))
    cuts = [0, 0] + cuts[1:] if seed % 2 else cuts     # an empty range too
    parts = [partial_state(s[a:b], v[a:b], vis[a:b]) for a, b in zip(cuts, cuts[1:])]
    for order in (parts, parts[::-1], [parts[i] for i in rng.permutation(len(parts))]):
        r = merge_states(order)
        assert np.max(np.abs(r["o"] - o_ref)) < 1e-12
        assert abs(r["lse"] - lse_ref) < 1e-12


def test_merge_of_empty_and_distant_states():
    """A state with no visible key changes nothing; if no state has one the
    row is fully masked (o = 0, lse = -inf); states whose maxima are 2000
    apart merge without overflow, the lower one contributing exp(-2000) = 0."""
    v = np.array([[1.0, 2.0], [3.0, -1.0]])
    full = partial_state([0.5, 1.5], v)
    empty = partial_state([0.5, 1.5], v, [False, False])
    assert empty["m"] == -math.inf and empty["l"] == 0.0 and np.all(empty["o_tilde"] == 0)
    o_ref, lse_ref = oracle.attn_from_scores(np.array([0.5, 1.5]), v.astype(np.float32))
    for parts in ([full, empty], [empty, full], [empty, full, empty]):
        r = merge_states(parts)
        assert np.max(np.abs(r["o"] - o_ref)) < 1e-14 and abs(r["lse"] - lse_ref) < 1e-14
    r = merge_states([empty, empty])
    assert np.all(r["o"] == 0) and r["lse"] == -math.inf
    far = partial_state([2000.0, 1999.0], v)
    r = merge_states([full, far])
    o_far, lse_far = oracle.attn_from_scores(np.array([2000.0, 1999.0]), v.astype(np.float32))
    assert np.all(np.isfinite(r["o"])) and np.max(np.abs(r["o"] - o_far)) < 1e-14
    assert abs(r["lse"] - lse_far) < 1e-12
