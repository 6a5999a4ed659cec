"""Block-sparse attention: the definition with a block mask, float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "Paper Notes: FlashAttention" page ("Experiments & Results") reports a
block-sparse variant of the method, 2-4x faster than dense FlashAttention in
proportion to the sparsity; it gives no further detail.  Reading taken here
(the plainest one consistent with the tiled method, which works block by
block):

* a block mask M of shape [ceil(N / block), ceil(N / block)] over the score
  matrix; query i may attend key j only when M[i // block, j // block] is
  nonzero (and, with ``causal``, when also j <= i);
* masked scores count as -inf, exactly like the causal mask: the result is
  the exact softmax over the allowed keys of each row;
* a row with no allowed key at all has O = 0 and LSE = -inf, and its
  gradients are zero (it receives and contributes nothing).

The arithmetic is the definition of ``oracle.attention`` with a general
boolean mask: S = scale Q K^T, masked entries -inf, P = softmax(S) per row,
O = P V, LSE = m + ln(l); backward dV = P^T dO, dP = dO V^T,
D_i = sum_j P_ij dP_ij, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
"""

import numpy as np

__all__ = [
    "allowed_mask",
    "forward_head_masked",
    "backward_head_masked",
    "forward_blocksparse",
    "backward_blocksparse",
]


def allowed_mask(n, block_mask, block, causal):
    """Boolean [n, n]: True where query i may attend key j."""
    bm = np.asarray(block_mask) != 0
    nb = (n + block - 1) // block
    assert bm.shape == (nb, nb), (bm.shape, nb)
    idx = np.arange(n) // block
    a = bm[idx[:, None], idx[None, :]]
    if causal:
        a = a & (np.arange(n)[None, :] <= np.arange(n)[:, None])
    return a


def _masked_softmax(s, allowed):
    """Row softmax over the allowed entries; (P, LSE) with P = 0 and
    LSE = -inf on rows that allow nothing."""
    s = np.where(allowed, s, -np.inf)
    any_row = allowed.any(axis=-1)
    m = np.where(any_row, np.max(np.where(allowed, s, -np.inf), axis=-1), 0.0)
    f = np.where(allowed, np.exp(s - m[:, None]), 0.0)
    l = f.sum(axis=-1)
    p = np.where(any_row[:, None], f / np.where(any_row, l, 1.0)[:, None], 0.0)
    lse = np.where(any_row, m + np.log(np.where(any_row, l, 1.0)), -np.inf)
    return p, lse


def forward_head_masked(q, k, v, allowed, scale):
    """O and LSE for one head under a boolean mask of allowed (query, key)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = (q @ k.T) * scale
    p, lse = _masked_softmax(s, allowed)
    return p @ v, lse


def backward_head_masked(q, k, v, do, allowed, scale):
    """dQ, dK, dV for one head under a boolean mask of allowed pairs."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = (q @ k.T) * scale
    p, _ = _masked_softmax(s, allowed)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1, keepdims=True)
    ds = p * (dp - dsum)
    return scale * (ds @ k), scale * (ds.T @ q), dv


def _head_mask(block_mask, b, h):
    bm = np.asarray(block_mask)
    return bm if bm.ndim == 2 else bm[b, h]


def forward_blocksparse(q, k, v, block_mask, causal=False, scale=None, block=128):
    """Batched forward over [B, H, N, d]; ``block_mask`` is [nb, nb] (shared by
    every head) or [B, H, nb, nb].  Returns (O, LSE)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b_, h_, n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(v)
    lse = np.empty((b_, h_, n))
    for b in range(b_):
        for h in range(h_):
            a = allowed_mask(n, _head_mask(block_mask, b, h), block, causal)
            o[b, h], lse[b, h] = forward_head_masked(q[b, h], k[b, h], v[b, h], a, scale)
    return o, lse


def backward_blocksparse(q, k, v, do, block_mask, causal=False, scale=None, block=128):
    """Batched backward over [B, H, N, d]; returns (dQ, dK, dV)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b_, h_, n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(b_):
        for h in range(h_):
            a = allowed_mask(n, _head_mask(block_mask, b, h), block, causal)
            dq[b, h], dk[b, h], dv[b, h] = backward_head_masked(q[b, h], k[b, h], v[b, h], do[b, h], a, scale)
    return dq, dk, dv
