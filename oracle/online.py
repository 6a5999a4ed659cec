"""The pages' tiled online-softmax forward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the loop the pages describe -- queries in row blocks, keys and values
streamed past them in column blocks, a running max ``m``, running sum ``l``
and unnormalised running output ``acc`` per query row, each rescaled by
exp(m - m_new) when the max grows, and a single division by ``l`` at the end:

* "flash attention" page, "build it from scratch" (the block loop with Bq/Bk);
* aicassindra page, "Rescale and accumulate: the forward pass in one loop"
  and "Online softmax: the running-max, running-sum idea";
* "Paper Notes: FlashAttention", "Tiling: Block-by-Block Softmax" (the
  two-block merge rule for m and l).

Reading of a garble: the pseudocode on the Paper Notes page ("The Complete
Algorithm in Pseudocode", its step 4) divides each block's contribution by the
running sum of that moment and then rescales the accumulator by the old-max
factor alone, which mixes terms normalised by different sums; it does not
reproduce the one-shot softmax.  The other two pages accumulate unnormalised
and divide once at the end; that is the form used here.

Two additions the pages leave open: the explicit ``scale`` and ``causal`` of
:mod:`oracle.attention`, and the guard for a block in which a row sees only
masked (-inf) scores -- while the running max is still -inf the rescale factor
is taken as 1 and the block's probabilities as 0, so no 0/0 appears.

Its purpose is to pin :mod:`oracle.attention` (tiled == one-shot for every
block size) and to replay the pages' worked examples step by step.
"""

import numpy as np

__all__ = ["flash_forward_head", "online_trace"]


def _merge_block(m, l, acc, s, v_blk):
    """Fold one block of scores ``s`` [rows, cols] and values into (m, l, acc)."""
    m_new = np.maximum(m, np.max(s, axis=-1))
    live = np.isfinite(m_new)
    m_safe = np.where(live, m_new, 0.0)
    p = np.where(live[:, None], np.exp(s - m_safe[:, None]), 0.0)
    a = np.where(live, np.exp(np.where(live, m - m_safe, 0.0)), 1.0)
    l = a * l + np.sum(p, axis=-1)
    acc = a[:, None] * acc + p @ v_blk
    return m_new, l, acc


def flash_forward_head(q, k, v, causal=False, scale=None, block_q=64, block_k=64):
    """O and LSE of one head by the block loop; ``q, k, v`` are [N, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, block_q):
        qi = q[i0 : i0 + block_q]
        rows = np.arange(i0, i0 + qi.shape[0])
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], v.shape[1]))
        for j0 in range(0, n, block_k):
            kj = k[j0 : j0 + block_k]
            vj = v[j0 : j0 + block_k]
            s = (qi @ kj.T) * scale
            if causal:
                cols = np.arange(j0, j0 + kj.shape[0])
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m, l, acc = _merge_block(m, l, acc, s, vj)
        o[i0 : i0 + qi.shape[0]] = acc / l[:, None]
        lse[i0 : i0 + qi.shape[0]] = m + np.log(l)
    return o, lse


def online_trace(score_blocks):
    """Running (m, l) of one score row after each block, in the pages' order.

    ``score_blocks`` is a list of 1-D arrays (the blocks of one row of S).
    Returns a list of ``(m, l, rescale)`` tuples where ``rescale`` is the
    factor exp(m_old - m_new) applied to the earlier sum when that block
    arrived (1.0 for the first block).
    """
    m = -np.inf
    l = 0.0
    out = []
    for blk in score_blocks:
        blk = np.asarray(blk, dtype=np.float64)
        m_new = max(m, float(np.max(blk)))
        a = 1.0 if m == -np.inf else float(np.exp(m - m_new))
        l = a * l + float(np.sum(np.exp(blk - m_new)))
        m = m_new
        out.append((m, l, a))
    return out
