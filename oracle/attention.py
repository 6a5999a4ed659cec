"""The definition of exact attention and its gradients, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Conventions shared by every function:

* ``q, k, v, do`` are float64 arrays of shape ``[B, H, N, d]`` (or ``[N, d]``
  for the per-head helpers).  Queries and keys share the length ``N``.
* ``scale`` multiplies the scores before the softmax.  The "Paper Notes:
  FlashAttention" page ("What Are We Computing?") writes S = Q K^T with no
  scale; the "flash attention" page ("build it from scratch") divides by
  sqrt(d).  Reading: the scale is an explicit argument; callers pass
  1/sqrt(d) for the usual attention and 1 to reproduce the unscaled examples.
* ``causal``: query i may attend key j only when j <= i (the lower triangle
  including the diagonal).  The aicassindra page ("Common pitfalls") requires
  the mask but fixes no convention; with equal query and key lengths the
  top-left and bottom-right alignments coincide.
* The saved softmax statistic is LSE_i = m_i + ln(l_i) (natural log), which
  packs the pages' per-row pair (m, l) ("Background", "Key Ideas" on the
  Paper Notes page; "The backward pass" on the aicassindra page) into one
  number: softmax_ij = exp(S_ij - LSE_i).

Everything is evaluated as written: S and P are materialised for a whole head
(or for a block of whole rows at a time in the ``*_rows`` helpers, which is
the same definition restricted to those rows -- rows of a softmax do not
interact).
"""

import numpy as np

__all__ = [
    "scores",
    "softmax_rows",
    "forward_head",
    "forward",
    "backward_head",
    "backward",
    "forward_rows",
    "head_row_stats",
    "backward_query_rows",
    "backward_key_rows",
]


def _f64(x):
    a = np.asarray(x, dtype=np.float64)
    return a


def scores(q, k, scale, causal):
    """S = scale * Q K^T for one head, with the causal mask applied as -inf.

    "Paper Notes: FlashAttention", "What Are We Computing?": S = Q K^T (N x N).
    "flash attention", "build it from scratch": the 1/sqrt(d) factor.
    """
    q = _f64(q)
    k = _f64(k)
    s = (q @ k.T) * scale
    if causal:
        n_q, n_k = s.shape
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def softmax_rows(s):
    """Numerically stable row softmax, returning (P, m, l).

    "Paper Notes: FlashAttention", "Tiling: Block-by-Block Softmax":
    m(x) = max_i x_i, f(x) = exp(x - m(x)), l(x) = sum f(x),
    softmax(x) = f(x) / l(x).
    """
    m = np.max(s, axis=-1, keepdims=True)
    f = np.exp(s - m)
    l = np.sum(f, axis=-1, keepdims=True)
    return f / l, m[..., 0], l[..., 0]


def forward_head(q, k, v, causal=False, scale=None):
    """O and LSE for one head: S = scale Q K^T, P = softmax(S), O = P V.

    "Paper Notes: FlashAttention", "What Are We Computing?" (the three-line
    definition); the row statistics are those of "Tiling: Block-by-Block
    Softmax"; LSE = m + ln(l).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = p @ v
    lse = m + np.log(l)
    return o, lse


def forward(q, k, v, causal=False, scale=None):
    """Batched :func:`forward_head` over ``[B, H, N, d]``; returns (O, LSE)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, h_, n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((b_, h_, n, v.shape[-1]))
    lse = np.empty((b_, h_, n))
    for b in range(b_):
        for h in range(h_):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def backward_head(q, k, v, do, causal=False, scale=None):
    """dQ, dK, dV for one head by the chain rule through the definition.

    The pages leave the gradient formulas to a companion article (aicassindra
    page, "The backward pass: recompute instead of store"); these are the
    textbook vector-Jacobian products of L = sum(dO * O) through
    S = scale Q K^T, P = softmax(S), O = P V:

        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D 1^T)          (masked entries have P = 0, so dS = 0)
        dQ = scale dS K,  dK = scale dS^T Q
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, _, _ = softmax_rows(s)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1, keepdims=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, causal=False, scale=None):
    """Batched :func:`backward_head` over ``[B, H, N, d]``; returns (dQ, dK, dV)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, h_, n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(b_):
        for h in range(h_):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], causal, scale
            )
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Row-restricted forms of the same definition, for sequences too long to hold
# a whole N x N head in memory.  Each evaluates the formulas above for the
# requested rows only (rows of S and P are independent of one another).
# ---------------------------------------------------------------------------


def _causal_row_scores(q_rows, k, rows, scale, causal):
    s = (q_rows @ k.T) * scale
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > np.asarray(rows)[:, None], -np.inf, s)
    return s


def forward_rows(q, k, v, rows, causal=False, scale=None):
    """O and LSE of the listed query rows of one head (``q, k, v`` are [N, d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    rows = np.asarray(rows, dtype=np.int64)
    s = _causal_row_scores(q[rows], k, rows, scale, causal)
    p, m, l = softmax_rows(s)
    return p @ v, m + np.log(l)


def backward_query_rows(q, k, v, do, rows, causal=False, scale=None):
    """dQ of the listed query rows of one head.

    dQ_i needs only row i of P and dP: dQ_i = scale sum_j P_ij (dP_ij - D_i) K_j
    with D_i = sum_j P_ij dP_ij.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    rows = np.asarray(rows, dtype=np.int64)
    s = _causal_row_scores(q[rows], k, rows, scale, causal)
    p, _, _ = softmax_rows(s)
    dp = do[rows] @ v.T
    dsum = np.sum(p * dp, axis=-1, keepdims=True)
    ds = p * (dp - dsum)
    return scale * (ds @ k)


def head_row_stats(q, k, v, do, causal=False, scale=None, chunk=1024):
    """LSE_i and D_i = sum_j P_ij dP_ij for every query row of one head.

    Evaluated a block of whole rows at a time so that only ``chunk x N`` of S
    exists at once.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    lse = np.empty(n)
    dsum = np.empty(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        kk = k[: rows[-1] + 1] if causal else k
        vv = v[: rows[-1] + 1] if causal else v
        s = _causal_row_scores(q[rows], kk, rows, scale, causal)
        p, m, l = softmax_rows(s)
        lse[rows] = m + np.log(l)
        dp = do[rows] @ vv.T
        dsum[rows] = np.sum(p * dp, axis=-1)
    return lse, dsum


def backward_key_rows(q, k, v, do, cols, lse, dsum, causal=False, scale=None, chunk=4096):
    """dK and dV of the listed key rows of one head.

    Uses P_ij = exp(S_ij - LSE_i) (the softmax definition written with the
    row log-sum-exp) and D_i from :func:`head_row_stats`:
    dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i P_ij (dP_ij - D_i) Q_i.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, k.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    i0 = int(cols.min()) if causal else 0
    for r0 in range(i0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        st = (q[rows] @ k[cols].T) * scale  # [rows, cols]
        if causal:
            st = np.where(cols[None, :] > rows[:, None], -np.inf, st)
        p = np.exp(st - lse[rows][:, None])
        dp = do[rows] @ v[cols].T
        ds = p * (dp - dsum[rows][:, None])
        dv += p.T @ do[rows]
        dk += scale * (ds.T @ q[rows])
    return dk, dv
