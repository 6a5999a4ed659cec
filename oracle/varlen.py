"""Attention with unequal query and key lengths, and the merge of partial
results over key splits, float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Queries [Nq, d], keys and values [Nk, d].  Non-causal: every query sees
  every key.  Causal, with Nq != Nk, the pages fix no alignment ("Common
  pitfalls" on the aicassindra page only requires the mask).  Reading taken:
  bottom-right alignment, the one of a query block appended after Nk - Nq
  earlier tokens (decoding, chunked prefill): query i sees key j when
  j <= i + (Nk - Nq).  With Nq == Nk it is the square causal mask.  When
  Nq > Nk the first Nq - Nk rows see no key: O = 0, LSE = -inf (as for the
  empty rows of the block-sparse variant).
* Split-K/V: the keys are cut into consecutive chunks, each chunk gives per
  row the statistics (m, l) of its scores and the unnormalised product
  sum_j exp(S_ij - m) V_j, and the chunks are combined by the two-block rule
  of "Tiling: Block-by-Block Softmax" (Paper Notes): m = max(m1, m2),
  l = exp(m1 - m) l1 + exp(m2 - m) l2, and the same weights on the products.
  The result equals the one-shot definition.
"""

import numpy as np

from oracle import blocksparse as _bs

__all__ = [
    "allowed_qk",
    "forward_qk",
    "backward_qk",
    "partial_stats",
    "merge_two",
    "finish",
    "forward_qk_batched",
    "backward_qk_batched",
]


def allowed_qk(nq, nk, causal):
    """Boolean [nq, nk]: query i may attend key j."""
    a = np.ones((nq, nk), dtype=bool)
    if causal:
        a = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq)
    return a


def forward_qk(q, k, v, causal, scale):
    """O [nq, d] and LSE [nq] for one head (definition, with the mask above)."""
    a = allowed_qk(q.shape[0], k.shape[0], causal)
    return _bs.forward_head_masked(q, k, v, a, scale)


def backward_qk(q, k, v, do, causal, scale):
    """dQ, dK, dV for one head."""
    a = allowed_qk(q.shape[0], k.shape[0], causal)
    return _bs.backward_head_masked(q, k, v, do, a, scale)


def partial_stats(q, k, v, scale, allowed):
    """Per-row (m, l, acc) over one chunk of keys: m the max allowed score (or
    -inf), l = sum of exp(S - m) over allowed keys, acc = sum exp(S - m) V."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    m = np.max(s, axis=-1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    f = np.where(allowed & live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
    return m, f.sum(axis=-1), f @ v


def merge_two(p1, p2):
    """The two-block rule on (m, l, acc) per row; rows that saw nothing in one
    chunk (m = -inf) take the other chunk's statistics unchanged."""
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    m = np.maximum(m1, m2)
    safe = np.where(np.isfinite(m), m, 0.0)
    w1 = np.where(np.isfinite(m1), np.exp(m1 - safe), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(m2 - safe), 0.0)
    return m, w1 * l1 + w2 * l2, w1[:, None] * a1 + w2[:, None] * a2


def finish(stats):
    """(O, LSE) from merged (m, l, acc): O = acc / l, LSE = m + ln l; rows that
    saw no key get O = 0 and LSE = -inf."""
    m, l, acc = stats
    live = l > 0
    o = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
    lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def forward_qk_batched(q, k, v, causal=False, scale=None):
    """Over [B, H, Nq, d] queries and [B, H, Nk, d] keys / values."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b_, h_, nq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    lse = np.empty((b_, h_, nq))
    for b in range(b_):
        for h in range(h_):
            o[b, h], lse[b, h] = forward_qk(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def backward_qk_batched(q, k, v, do, causal=False, scale=None):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b_, h_, nq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(b_):
        for h in range(h_):
            dq[b, h], dk[b, h], dv[b, h] = backward_qk(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale)
    return dq, dk, dv
