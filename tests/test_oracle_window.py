"""Pins of oracle.window (causal sliding window) against independent routines.

* A window of N keys or more is the plain causal definition.
* Window 1: each row sees only its own key, so O = V, LSE_i = scale q_i . k_i,
  dQ = dK = 0 (a softmax over one entry does not move) and dV = dO.
* Row by row: row i is the plain attention of q_i over keys
  max(0, i - W + 1) .. i alone (oracle.attention.forward_head on the slice),
  and dQ_i is that row problem's gradient.
* Finite differences of the masked loss for all three gradients.
A planted off-by-one (a window one key wider) fails the row-by-row pin.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import window as W


def _inputs(seed, shape):
    r = np.random.default_rng(seed)
    return [r.standard_normal(shape) for _ in range(4)]


def test_wide_window_is_the_causal_definition():
    q, k, v, do = _inputs(1, (1, 2, 19, 8))
    for win in (19, 50):
        o, lse = W.forward_window(q, k, v, win, 0.3)
        o_r, lse_r = A.forward(q, k, v, True, 0.3)
        np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_r, rtol=0, atol=1e-12)
        for x, y in zip(W.backward_window(q, k, v, do, win, 0.3), A.backward(q, k, v, do, True, 0.3)):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-11)


def test_window_one_is_the_identity_on_values():
    q, k, v, do = _inputs(2, (2, 1, 13, 4))
    o, lse = W.forward_window(q, k, v, 1, 0.7)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * np.sum(q * k, axis=-1), rtol=0, atol=1e-13)
    dq, dk, dv = W.backward_window(q, k, v, do, 1, 0.7)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-14)


@pytest.mark.parametrize("win", [2, 5, 16])
def test_rows_are_attention_over_their_window(win):
    q, k, v, do = _inputs(3 + win, (1, 1, 21, 6))
    o, lse = W.forward_window(q, k, v, win, 0.5)
    dq, _, _ = W.backward_window(q, k, v, do, win, 0.5)
    for i in range(21):
        lo = max(0, i - win + 1)
        o_r, lse_r = A.forward_head(q[0, 0, i:i + 1], k[0, 0, lo:i + 1], v[0, 0, lo:i + 1], False, 0.5)
        np.testing.assert_allclose(o[0, 0, i], o_r[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0, i], lse_r[0], rtol=0, atol=1e-12)
        dq_r, _, _ = A.backward_head(q[0, 0, i:i + 1], k[0, 0, lo:i + 1], v[0, 0, lo:i + 1], do[0, 0, i:i + 1],
                                     False, 0.5)
        np.testing.assert_allclose(dq[0, 0, i], dq_r[0], rtol=0, atol=1e-12)


def test_gradients_match_finite_differences():
    q, k, v, do = _inputs(9, (1, 1, 7, 3))
    win, scale = 3, 0.9

    def loss(qq, kk, vv):
        o, _ = W.forward_window(qq, kk, vv, win, scale)
        return float(np.sum(o * do))

    grads = W.backward_window(q, k, v, do, win, scale)
    eps = 1e-6
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


def test_planted_wider_window_fails(monkeypatch):
    real = W.allowed_window
    monkeypatch.setattr(W, "allowed_window", lambda n, win: real(n, win + 1))
    q, k, v, _ = _inputs(11, (1, 1, 12, 4))
    o, _ = W.forward_window(q, k, v, 4, 0.5)
    i, lo = 9, 6
    o_r, _ = A.forward_head(q[0, 0, i:i + 1], k[0, 0, lo:i + 1], v[0, 0, lo:i + 1], False, 0.5)
    assert np.max(np.abs(o[0, 0, i] - o_r[0])) > 1e-3
