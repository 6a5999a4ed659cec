"""Attention with dropout on the probabilities, float64, CPU, and the
counter-based generator that draws the dropout mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name dropout and masking among the element-wise operations that
kernel fusion folds into one kernel ("Background", Paper Notes); they fix no
formula.  Readings taken:

* Placement: dropout acts on the normalised probabilities before the product
  with V (the usual attention dropout).  With Z_ij in {0, 1} kept with
  probability 1 - p and s = 1 / (1 - p):
      O = (P * Z) V s,   LSE unchanged (the statistics of S, from which the
      backward pass recomputes P),
      dV = (P * Z)^T dO s,   dP = (dO V^T) * Z s,
      D_i = sum_j P_ij dP_ij = sum_k dO_ik O_ik  (still; O carries Z s),
      dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
* Generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter
  (c0, c1, c2, c3) and a 64-bit key (k0, k1); each round multiplies c0 and c2
  by 0xD2511F53 and 0xCD9E8D57 (full 64-bit products), and sets
  (c0, c1, c2, c3) <- (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1,
  lo(c0 M0)); the key gains (0x9E3779B9, 0xBB67AE85) before every round but
  the first.
* Which random word decides which element: for head index bh = b H + h,
  query i and key j, the counter is (j >> 2, i, bh, offset) and the key
  (seed mod 2^32, seed >> 32); the four output words belong to keys
  4 (j >> 2) + 0..3.  The element is kept when its word u satisfies
  u >= t with t = min(floor(p 2^32), 2^32 - 1), p the float32 value of the
  dropout probability (so p = 0 keeps everything).
"""

import numpy as np

from oracle import attention as _A

__all__ = [
    "philox4x32_10",
    "threshold",
    "keep_mask",
    "forward_head",
    "backward_head",
    "forward",
    "backward",
]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on arrays of 32-bit values (any broadcastable shapes);
    returns the four output words as uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & _MASK)
    k1 = np.uint64(int(k1) & _MASK)
    m0, m1, mask = np.uint64(_M0), np.uint64(_M1), np.uint64(_MASK)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + _W0) & _MASK)
            k1 = np.uint64((int(k1) + _W1) & _MASK)
        p0 = c0 * m0  # < 2^64: exact in uint64
        p1 = c2 * m1
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & mask, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & mask)
    return c0, c1, c2, c3


def threshold(p):
    """Integer keep threshold of a dropout probability (float32 value of p)."""
    pf = float(np.float32(p))
    return min(int(np.floor(pf * 4294967296.0)), 4294967295)


def keep_mask(bh, nq, nk, p, seed, offset=0):
    """Boolean [nq, nk]: element (i, j) of head bh is kept."""
    i = np.arange(nq, dtype=np.uint64)[:, None]
    j = np.arange(nk, dtype=np.uint64)[None, :]
    words = philox4x32_10(j >> np.uint64(2), i, np.uint64(bh), np.uint64(offset & _MASK), seed & _MASK,
                          (seed >> 32) & _MASK)
    jm = (j & np.uint64(3)).astype(np.int64)
    u = np.choose(np.broadcast_to(jm, (nq, nk)), [np.broadcast_to(w, (nq, nk)) for w in words])
    return u >= np.uint64(threshold(p))


def _probs(q, k, causal, scale):
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    s = (q @ k.T) * scale
    if causal:
        n = s.shape[0]
        s = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    lse = (m + np.log(e.sum(axis=-1, keepdims=True)))[:, 0]
    return e / e.sum(axis=-1, keepdims=True), lse


def forward_head(q, k, v, causal, scale, z, p):
    """O and LSE for one head with keep mask z (bool [n, n]) and probability p."""
    P, lse = _probs(q, k, causal, scale)
    s = 1.0 / (1.0 - float(np.float32(p)))
    return (P * z) @ np.asarray(v, dtype=np.float64) * s, lse


def backward_head(q, k, v, do, causal, scale, z, p):
    """dQ, dK, dV for one head (the vector-Jacobian product of the forward
    above with the mask held fixed)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    P, _ = _probs(q, k, causal, scale)
    s = 1.0 / (1.0 - float(np.float32(p)))
    Pd = P * z * s
    dv = Pd.T @ do
    dp = (do @ v.T) * z * s
    dsum = (P * dp).sum(axis=-1, keepdims=True)
    ds = P * (dp - dsum)
    return scale * ds @ k, scale * ds.T @ q, dv


def forward(q, k, v, causal, scale, p, seed, offset=0):
    """[B, H, N, d] -> (O, LSE), masks from the generator."""
    q = np.asarray(q, dtype=np.float64)
    b_, h_, n, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((b_, h_, n))
    for b in range(b_):
        for h in range(h_):
            z = keep_mask(b * h_ + h, n, n, p, seed, offset)
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], causal, scale, z, p)
    return o, lse


def backward(q, k, v, do, causal, scale, p, seed, offset=0):
    q = np.asarray(q, dtype=np.float64)
    b_, h_, n, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    for b in range(b_):
        for h in range(h_):
            z = keep_mask(b * h_ + h, n, n, p, seed, offset)
            dq[b, h], dk[b, h], dv[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale, z, p)
    return dq, dk, dv


# The no-dropout definition is the plain oracle's; kept importable here for
# tests that compare the two.
plain_forward_head = _A.forward_head
plain_backward_head = _A.backward_head
