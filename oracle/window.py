"""Causal sliding-window attention: the definition with a banded mask,
float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A second mask of the kind the "Paper Notes: FlashAttention" page
("Background") lists among the element-wise operations fused into the
attention kernel: the causal mask restricted to the last ``window`` keys.
Reading taken here: query i attends key j exactly when i - window < j <= i
(window >= 1; a window of N or more keys is the plain causal mask).  Masked
scores count as -inf; every row keeps its own key, so no row is empty.  The
arithmetic is the masked definition of :mod:`oracle.blocksparse` with this
mask.
"""

import numpy as np

from oracle import blocksparse as _bs

__all__ = ["allowed_window", "forward_window", "backward_window"]


def allowed_window(n, window):
    """Boolean [n, n]: True where query i may attend key j."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & (j > i - int(window))


def forward_window(q, k, v, window, scale=None):
    """O and LSE for [B, H, N, d] inputs."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    allowed = allowed_window(N, window)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _bs.forward_head_masked(q[b, h], k[b, h], v[b, h], allowed, scale)
    return o, lse


def backward_window(q, k, v, do, window, scale=None):
    """dQ, dK, dV for [B, H, N, d] inputs under the window mask."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    allowed = allowed_window(N, window)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _bs.backward_head_masked(q[b, h], k[b, h], v[b, h], do[b, h], allowed,
                                                                     scale)
    return dq, dk, dv
