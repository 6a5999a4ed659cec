"""Key padding: the definition with a per-sequence key length, float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "Paper Notes: FlashAttention" page ("Background") lists the mask beside
dropout among the element-wise operations that kernel fusion folds into one
kernel, and fixes no particular mask.  Reading taken here: the key padding
mask of batched sequences of different lengths, the common form of an
attention mask.  Batch b holds key_len[b] valid keys (clamped to [0, N]); for
every head and query of that batch,

* key j is masked when j >= key_len[b] (and, with ``causal``, when j > i);
* masked scores count as -inf, exactly like the causal mask: each row's
  result is the exact softmax over its allowed keys;
* a row with no allowed key (key_len[b] = 0) has O = 0, LSE = -inf and zero
  gradients; padded keys receive dK = dV = 0.

The arithmetic is the masked definition of :mod:`oracle.blocksparse`
(S = scale Q K^T, masked entries -inf, P = softmax(S), O = P V; the textbook
backward), with this mask.
"""

import numpy as np

from oracle import blocksparse as _bs

__all__ = ["clamp_len", "allowed_keypad", "forward_keypad", "backward_keypad"]


def clamp_len(length, n):
    """A key length as the kernels read it: below 0 counts as 0, above n as n."""
    return int(min(max(int(length), 0), n))


def allowed_keypad(n, length, causal):
    """Boolean [n, n]: True where query i may attend key j."""
    length = clamp_len(length, n)
    j = np.arange(n)
    a = np.broadcast_to(j[None, :] < length, (n, n))
    if causal:
        a = a & (j[None, :] <= j[:, None])
    return np.array(a)


def forward_keypad(q, k, v, key_len, causal=False, scale=None):
    """O and LSE for [B, H, N, d] inputs; key_len has one entry per batch."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        allowed = allowed_keypad(N, key_len[b], causal)
        for h in range(H):
            o[b, h], lse[b, h] = _bs.forward_head_masked(q[b, h], k[b, h], v[b, h], allowed, scale)
    return o, lse


def backward_keypad(q, k, v, do, key_len, causal=False, scale=None):
    """dQ, dK, dV for [B, H, N, d] inputs under the key padding mask."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        allowed = allowed_keypad(N, key_len[b], causal)
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _bs.backward_head_masked(q[b, h], k[b, h], v[b, h], do[b, h], allowed,
                                                                     scale)
    return dq, dk, dv
