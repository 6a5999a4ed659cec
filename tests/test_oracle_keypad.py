"""Pins of oracle.keypad (key padding) against independent routines.

* With every key valid the padded definition is the plain one
  (oracle.attention.forward / backward).
* Full mask, key length L: every row is the plain attention of the query
  against the first L keys alone (oracle.attention.forward_head /
  backward_head on the sliced keys), and the padded keys get zero gradients.
* Causal, key length L: rows i < L are the plain causal attention of the
  first L tokens; rows i >= L see exactly keys 0 .. L - 1.
* Length 0: O = 0, LSE = -inf, zero gradients; lengths outside [0, N] clamp.
* Finite differences of the masked loss for the gradients on a tiny case.
A planted off-by-one in the mask (j <= L) fails the slicing pins.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import keypad as KP


def _inputs(seed, shape):
    r = np.random.default_rng(seed)
    return [r.standard_normal(shape) for _ in range(4)]


def test_full_length_is_the_plain_definition():
    q, k, v, do = _inputs(1, (2, 2, 23, 8))
    for causal in (False, True):
        o, lse = KP.forward_keypad(q, k, v, [23, 40], causal, 0.3)
        o_r, lse_r = A.forward(q, k, v, causal, 0.3)
        np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_r, rtol=0, atol=1e-12)
        g = KP.backward_keypad(q, k, v, do, [23, 40], causal, 0.3)
        g_r = A.backward(q, k, v, do, causal, 0.3)
        for x, y in zip(g, g_r):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-11)


@pytest.mark.parametrize("length", [1, 7, 16, 22])
def test_full_mask_equals_sliced_keys(length):
    q, k, v, do = _inputs(2 + length, (1, 2, 23, 8))
    o, lse = KP.forward_keypad(q, k, v, [length], False, 0.4)
    dq, dk, dv = KP.backward_keypad(q, k, v, do, [length], False, 0.4)
    for h in range(2):
        L = length
        o_r, lse_r = A.forward_head(q[0, h], k[0, h, :L], v[0, h, :L], False, 0.4)
        np.testing.assert_allclose(o[0, h], o_r, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], lse_r, rtol=0, atol=1e-12)
        dq_r, dk_r, dv_r = A.backward_head(q[0, h], k[0, h, :L], v[0, h, :L], do[0, h], False, 0.4)
        np.testing.assert_allclose(dq[0, h], dq_r, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[0, h, :L], dk_r, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[0, h, :L], dv_r, rtol=0, atol=1e-11)
        assert np.all(dk[0, h, L:] == 0) and np.all(dv[0, h, L:] == 0)


@pytest.mark.parametrize("length", [1, 9, 22])
def test_causal_rows_split_at_the_length(length):
    q, k, v, _ = _inputs(30 + length, (1, 1, 23, 8))
    o, lse = KP.forward_keypad(q, k, v, [length], True, 0.5)
    L = length
    o_top, lse_top = A.forward_head(q[0, 0, :L], k[0, 0, :L], v[0, 0, :L], True, 0.5)
    np.testing.assert_allclose(o[0, 0, :L], o_top, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, :L], lse_top, rtol=0, atol=1e-12)
    o_low, lse_low = A.forward_head(q[0, 0, L:], k[0, 0, :L], v[0, 0, :L], False, 0.5)
    np.testing.assert_allclose(o[0, 0, L:], o_low, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, L:], lse_low, rtol=0, atol=1e-12)


def test_empty_and_clamped_lengths():
    q, k, v, do = _inputs(5, (3, 1, 11, 4))
    o, lse = KP.forward_keypad(q, k, v, [0, -5, 99], True, 0.7)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    o_r, lse_r = A.forward(q[2:], k[2:], v[2:], True, 0.7)
    np.testing.assert_allclose(o[2:], o_r, rtol=0, atol=1e-12)
    dq, dk, dv = KP.backward_keypad(q, k, v, do, [0, -5, 99], True, 0.7)
    for g in (dq, dk, dv):
        assert np.all(g[:2] == 0)


def test_gradients_match_finite_differences():
    q, k, v, do = _inputs(7, (1, 1, 6, 3))
    L, scale = 4, 0.8

    def loss(qq, kk, vv):
        o, _ = KP.forward_keypad(qq, kk, vv, [L], True, scale)
        return float(np.sum(o * do))

    dq, dk, dv = KP.backward_keypad(q, k, v, do, [L], True, scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


def test_planted_off_by_one_fails(monkeypatch):
    real = KP.allowed_keypad

    def wrong(n, length, causal):
        a = real(n, min(KP.clamp_len(length, n) + 1, n), causal)
        return a

    monkeypatch.setattr(KP, "allowed_keypad", wrong)
    q, k, v, _ = _inputs(9, (1, 1, 12, 4))
    o, _ = KP.forward_keypad(q, k, v, [5], False, 0.5)
    o_r, _ = A.forward_head(q[0, 0], k[0, 0, :5], v[0, 0, :5], False, 0.5)
    assert np.max(np.abs(o[0, 0] - o_r)) > 1e-3
