"""Softmax attention computed block by block with the two-block merge rule, in
float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The mathematics ("Paper Notes: FlashAttention", "Tiling: Block-by-Block
Softmax"): for a row of scores split into two parts x1 and x2,

    m(x) = max(m(x1), m(x2)),
    l(x) = e^(m(x1) - m) l(x1) + e^(m(x2) - m) l(x2),

and the unnormalised output sum_j e^(x_j - m) v_j of the whole row combines
the parts' sums with the same two weights.  So the softmax statistics of any
set of keys are a triple state = (m, l, u) -- max score, sum of
exponentials relative to m, and the matching unnormalised output -- and the
rule above merges the states of two disjoint sets into the state of their
union.  The merge is associative, so the keys may be cut into any number of
parts of any sizes and the parts' states folded in any grouping; the result
is O = u / l and LSE = m + ln l, the one-shot softmax.  The running-max,
running-sum loop of the "flash attention" page ("build it from scratch") and
of the aicassindra page ("Online softmax: the running-max, running-sum idea",
"Rescale and accumulate") is the left-to-right fold of this rule; the
rescale factor it applies to the earlier sum is the first weight above.

Reading of a garble: the pseudocode on the Paper Notes page ("The Complete
Algorithm in Pseudocode", its step 4) divides each block's contribution by the
running sum of that moment and then rescales the accumulator by the old-max
factor alone, which mixes terms normalised by different sums; it does not
reproduce the one-shot softmax.  The merge rule keeps u unnormalised and
divides once at the end, as the other two pages do.

Additions the pages leave open: the explicit ``scale`` and ``causal`` of
:mod:`oracle.attention`, and rows of a part in which every score is masked
(-inf): such a part's state is (-inf, 0, 0), the identity of the merge (its
weight is taken as 0, never computed as e^(-inf - (-inf))).

Its purpose is to pin :mod:`oracle.attention` (block-wise == one-shot for every
partition of the keys) and to replay the pages' worked examples step by step.
"""

import numpy as np

__all__ = ["part_state", "merge_states", "flash_forward_head", "online_trace"]


def part_state(s, v_part):
    """State (m, l, u) of one part of the keys for each query row.

    ``s`` holds the part's scores [rows, keys] (masked entries -inf) and
    ``v_part`` its value rows [keys, d]: m = row max, l = sum_j e^(s_j - m),
    u = sum_j e^(s_j - m) v_j; a row with every score masked gets (-inf, 0, 0).
    """
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1)
    seen = np.isfinite(m)
    e = np.exp(s - np.where(seen, m, 0.0)[:, None]) * seen[:, None]
    return m, np.sum(e, axis=-1), e @ v_part


def merge_states(a, b):
    """The two-block rule: the state of the union of two disjoint key sets."""
    (m1, l1, u1), (m2, l2, u2) = a, b
    m = np.maximum(m1, m2)
    live = np.isfinite(m)
    ref = np.where(live, m, 0.0)
    w1 = np.where(np.isfinite(m1), np.exp(np.where(np.isfinite(m1), m1, 0.0) - ref), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(np.where(np.isfinite(m2), m2, 0.0) - ref), 0.0)
    return m, w1 * l1 + w2 * l2, w1[:, None] * u1 + w2[:, None] * u2


def _key_parts(n, block_k, key_bounds):
    if key_bounds is not None:
        b = sorted(set(int(x) for x in key_bounds) | {0, n})
        return [(b[i], b[i + 1]) for i in range(len(b) - 1) if b[i] < b[i + 1]]
    return [(j, min(n, j + block_k)) for j in range(0, n, block_k)]


def flash_forward_head(q, k, v, causal=False, scale=None, block_q=64, block_k=64, key_bounds=None, tree=False):
    """O and LSE of one head from per-part states; ``q, k, v`` are [N, d].

    Query rows are taken ``block_q`` at a time.  The keys are cut into parts
    of ``block_k`` keys, or at the given ``key_bounds`` (any increasing cut
    points, so parts of uneven sizes); the parts' states are folded left to
    right with :func:`merge_states`, or pairwise as a balanced tree when
    ``tree`` is set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    parts = _key_parts(k.shape[0], block_k, key_bounds)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, block_q):
        rows = np.arange(i0, min(n, i0 + block_q))
        states = []
        for j0, j1 in parts:
            s = (q[rows] @ k[j0:j1].T) * scale
            if causal:
                s = np.where(np.arange(j0, j1)[None, :] > rows[:, None], -np.inf, s)
            states.append(part_state(s, v[j0:j1]))
        if tree:
            while len(states) > 1:
                states = [merge_states(states[i], states[i + 1]) if i + 1 < len(states) else states[i]
                          for i in range(0, len(states), 2)]
            m, l, u = states[0]
        else:
            m, l, u = states[0]
            for st in states[1:]:
                m, l, u = merge_states((m, l, u), st)
        o[rows] = u / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def online_trace(score_blocks):
    """Running (m, l) of one score row after each block, in the pages' order.

    ``score_blocks`` is a list of 1-D arrays (the blocks of one row of S).
    Returns a list of ``(m, l, rescale)`` tuples where ``rescale`` is the
    merge weight exp(m_old - m_new) of the earlier blocks' sum when that block
    arrived (1.0 for the first block).
    """
    state = None
    out = []
    for blk in score_blocks:
        blk = np.asarray(blk, dtype=np.float64)[None, :]
        new = part_state(blk, np.zeros((blk.shape[1], 1)))
        if state is None:
            rescale = 1.0
            state = new
        else:
            rescale = float(np.exp(state[0][0] - max(state[0][0], new[0][0])))
            state = merge_states(state, new)
        out.append((float(state[0][0]), float(state[1][0]), rescale))
    return out
