"""The online-softmax recurrence for one query row, in fp64, block by block.

TEST INFRASTRUCTURE ONLY: used by the test suite to check the pages' block-wise
traces and the claim that block size and traversal order do not change the
result.  The product path never imports anything under ``oracle/``.

It takes the pages' steps in their order and notation:

    init   m = -inf, l = 0, o~ = 0
    for each block B of keys (in the chosen traversal order):
        m_blk = max_{j in B} s_j
        m_new = max(m, m_blk)
        alpha = exp(m - m_new)                 rescale factor, <= 1
        p_j   = exp(s_j - m_new)               j in B
        l     = alpha * l  + sum_j p_j
        o~    = alpha * o~ + sum_j p_j v_j
        m     = m_new
    o = o~ / l

-- "2.2b: FlashAttention -- Online Softmax", section "The Complete Online
   Softmax Algorithm"; "The math of FlashAttention" (aicassindra), section
   "The block-wise update, and the full algorithm".

Masked keys get score -inf *before* the block maximum is taken ("The math of
FlashAttention", "Pitfalls in implementing the recurrence"), so they add
p = exp(-inf) = 0.  The pages never meet a block whose keys are all masked
while m is still -inf, where exp(m - m_new) would be exp(-inf + inf); the
reading used here is that such a block leaves the empty state unchanged
(alpha = 0, p = 0), which is what skipping it would do.  A row that ends with
l = 0 gets o = 0 and lse = -inf.

partial_state() and merge_states() give the same state for a set of keys
directly and combine the states of disjoint key sets: each state is rewritten
to the common base max(m_i) by the rescaling identity and the rewritten sums
add ("The math of FlashAttention", sections "The running state: a max, a
denominator, and an output", "The rescaling identity, derived" and "Proof of
exactness", where block size and traversal order never enter the result).  The
pages apply the identity to one running state and one new block; applying it to
two states is the reading used for key ranges processed apart.
"""

import math

import numpy as np


def _exp(x):
    return math.exp(x) if x != -math.inf else 0.0


def online_attention_row(scores, values=None, block=2, order=None, visible=None):
    """Run the recurrence over one row of precomputed scores.

    scores  : 1-D sequence of n scores (already scaled).
    values  : n x dv array of value rows, or None for the softmax state only.
    block   : number of keys per block (the last block may be shorter).
    order   : sequence of block indices giving the traversal order
              (default: first to last).
    visible : optional boolean sequence of n; False keys are masked.

    Returns a dict with o (dv-vector or None), m, l, lse and trace, a list with
    one entry per visited block holding that block's m_blk, m_new, alpha, p,
    and the state l and o~ after the block.
    """
    s = np.asarray(scores, dtype=np.float64).copy()
    n = s.shape[0]
    if visible is not None:
        vis = np.asarray(visible, dtype=bool)
        s[~vis] = -math.inf
    v = None if values is None else np.asarray(values, dtype=np.float64).reshape(n, -1)
    if block < 1:
        raise ValueError("block must be >= 1")
    nblocks = (n + block - 1) // block
    if order is None:
        order = range(nblocks)
    order = list(order)
    if sorted(order) != list(range(nblocks)):
        raise ValueError("order must be a permutation of the block indices")

    m = -math.inf
    l = 0.0
    o_t = None if v is None else np.zeros(v.shape[1], dtype=np.float64)
    trace = []
    for b in order:
        lo, hi = b * block, min(n, (b + 1) * block)
        s_blk = s[lo:hi]
        m_blk = float(np.max(s_blk))
        m_new = max(m, m_blk)
        if m_new == -math.inf:
            # every key so far is masked: nothing to add, nothing to rescale
            alpha = 0.0
            p = np.zeros(hi - lo)
        else:
            alpha = _exp(m - m_new)
            p = np.array([_exp(x - m_new) for x in s_blk])
        l = alpha * l + float(np.sum(p))
        if v is not None:
            o_t = alpha * o_t + p @ v[lo:hi]
        m = m_new
        trace.append({
            "block": b, "m_blk": m_blk, "m_new": m_new, "alpha": alpha,
            "p": p.copy(), "l": l, "o_tilde": None if o_t is None else o_t.copy(),
        })

    if l == 0.0:
        o = None if v is None else np.zeros(v.shape[1])
        lse = -math.inf
    else:
        o = None if v is None else o_t / l
        lse = m + math.log(l)
    return {"o": o, "m": m, "l": l, "lse": lse, "trace": trace}


def partial_state(scores, values=None, visible=None):
    """The running state (m, l, o~) of one set of keys, from its definition.

    m is the largest visible score, l = sum_j exp(s_j - m) and
    o~ = sum_j exp(s_j - m) v_j over the visible keys ("The math of
    FlashAttention", "The running state: a max, a denominator, and an
    output").  With no visible key: m = -inf, l = 0, o~ = 0 (the state the
    recurrence starts from).

    Returns a dict with m, l and o_tilde (a dv-vector, or None without values).
    """
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    n = s.shape[0]
    vis = np.ones(n, dtype=bool) if visible is None else np.asarray(visible, dtype=bool)
    v = None if values is None else np.asarray(values, dtype=np.float64)
    if v is not None and v.ndim == 1:
        v = v[:, None]                                  # scalar values
    dv = None if v is None else v.shape[1]
    if not vis.any():
        return {"m": -math.inf, "l": 0.0, "o_tilde": None if v is None else np.zeros(dv)}
    m = float(np.max(s[vis]))
    w = np.where(vis, np.exp(np.where(vis, s - m, 0.0)), 0.0)
    return {"m": m, "l": float(np.sum(w)), "o_tilde": None if v is None else w @ v}


def merge_states(states):
    """Combine the states of disjoint key sets into the state of their union.

    states: a sequence of dicts with m, l and o_tilde (as partial_state
    returns).  The common base is M = max_i m_i; state i is rewritten to it by
    alpha_i = exp(m_i - M) <= 1, applied to both l_i and o~_i (the rescaling
    identity), and the rewritten sums add because the key sets are disjoint.
    States with no visible key (m = -inf) contribute nothing.  Returns a dict
    with m, l, o_tilde, o = o~ / l and lse = M + ln l; when no state has a
    visible key, o = 0 and lse = -inf.
    """
    states = list(states)
    if not states:
        raise ValueError("at least one state is needed")
    has_v = states[0]["o_tilde"] is not None
    dv = len(states[0]["o_tilde"]) if has_v else 0
    big_m = max(st["m"] for st in states)
    l = 0.0
    o_t = np.zeros(dv) if has_v else None
    if big_m != -math.inf:
        for st in states:
            alpha = _exp(st["m"] - big_m)
            l += alpha * st["l"]
            if has_v:
                o_t = o_t + alpha * np.asarray(st["o_tilde"], dtype=np.float64)
    if l == 0.0:
        return {"m": big_m, "l": 0.0, "o_tilde": o_t, "o": np.zeros(dv) if has_v else None,
                "lse": -math.inf}
    return {"m": big_m, "l": l, "o_tilde": o_t, "o": o_t / l if has_v else None,
            "lse": big_m + math.log(l)}
