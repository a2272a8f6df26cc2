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
