"""Pins of the block-sparse oracle (oracle/blocksparse.py).

Each check ties the masked definition to something other than itself: the
dense oracle (pinned in test_oracle.py) where the mask is all ones or is
implied by the causal mask, dense attention on independent sub-problems where
the mask makes heads of blocks independent, and central finite differences of
L = sum(dO * O) for the gradients.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import blocksparse as BS


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkvdo(n, d, seed):
    return tuple(_rand((n, d), seed + i) for i in range(4))


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_dense(causal):
    n, d, blk = 37, 5, 8
    q, k, v, do = _qkvdo(n, d, 1)
    nb = (n + blk - 1) // blk
    a = BS.allowed_mask(n, np.ones((nb, nb)), blk, causal)
    o, lse = BS.forward_head_masked(q, k, v, a, 0.4)
    o_ref, lse_ref = A.forward_head(q, k, v, causal, 0.4)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    g = BS.backward_head_masked(q, k, v, do, a, 0.4)
    g_ref = A.backward_head(q, k, v, do, causal, 0.4)
    for x, y in zip(g, g_ref):
        assert np.max(np.abs(x - y)) < 1e-12


def test_lower_block_triangle_with_causal_is_causal():
    # Blocks above the diagonal hold only keys j > i: masking them changes nothing.
    n, d, blk = 45, 4, 8
    q, k, v, do = _qkvdo(n, d, 2)
    nb = (n + blk - 1) // blk
    tri = np.tril(np.ones((nb, nb)))
    a = BS.allowed_mask(n, tri, blk, True)
    o, lse = BS.forward_head_masked(q, k, v, a, 0.5)
    o_ref, lse_ref = A.forward_head(q, k, v, True, 0.5)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12


def test_block_diagonal_mask_is_independent_blocks():
    # Each block of queries attends only its own block of keys: attention on
    # each diagonal block separately, and no gradient crosses blocks.
    n, d, blk = 29, 6, 8  # ragged last block (5 rows)
    q, k, v, do = _qkvdo(n, d, 3)
    nb = (n + blk - 1) // blk
    a = BS.allowed_mask(n, np.eye(nb), blk, False)
    o, lse = BS.forward_head_masked(q, k, v, a, 0.3)
    dq, dk, dv = BS.backward_head_masked(q, k, v, do, a, 0.3)
    for b in range(nb):
        sl = slice(b * blk, min(n, (b + 1) * blk))
        o_b, lse_b = A.forward_head(q[sl], k[sl], v[sl], False, 0.3)
        g_b = A.backward_head(q[sl], k[sl], v[sl], do[sl], False, 0.3)
        assert np.max(np.abs(o[sl] - o_b)) < 1e-12 and np.max(np.abs(lse[sl] - lse_b)) < 1e-12
        for x, y in zip((dq[sl], dk[sl], dv[sl]), g_b):
            assert np.max(np.abs(x - y)) < 1e-12


def test_first_key_block_only_is_truncated_attention():
    n, d, blk = 40, 5, 8
    q, k, v, do = _qkvdo(n, d, 4)
    nb = (n + blk - 1) // blk
    bm = np.zeros((nb, nb))
    bm[:, 0] = 1
    a = BS.allowed_mask(n, bm, blk, False)
    o, lse = BS.forward_head_masked(q, k, v, a, 0.7)
    o_ref, lse_ref = A.forward_head(q, k[:blk], v[:blk], False, 0.7)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    dq, dk, dv = BS.backward_head_masked(q, k, v, do, a, 0.7)
    # Same function of (Q, K[:blk], V[:blk]): identical gradients there, zero elsewhere.
    s = (q @ k[:blk].T) * 0.7
    p, _, _ = A.softmax_rows(s)
    dp = do @ v[:blk].T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    assert np.max(np.abs(dq - 0.7 * ds @ k[:blk])) < 1e-12
    assert np.max(np.abs(dk[:blk] - 0.7 * ds.T @ q)) < 1e-12 and np.all(dk[blk:] == 0)
    assert np.max(np.abs(dv[:blk] - p.T @ do)) < 1e-12 and np.all(dv[blk:] == 0)


def test_empty_rows():
    # A query block with no allowed key block: O = 0, LSE = -inf, no gradient;
    # the other rows are unaffected (rows of a softmax are independent).
    n, d, blk = 24, 4, 8
    q, k, v, do = _qkvdo(n, d, 5)
    bm = np.ones((3, 3))
    bm[1, :] = 0
    a = BS.allowed_mask(n, bm, blk, False)
    o, lse = BS.forward_head_masked(q, k, v, a, 0.5)
    assert np.all(o[8:16] == 0) and np.all(np.isneginf(lse[8:16]))
    keep = np.r_[0:8, 16:24]
    o_ref, lse_ref = A.forward_head(q[keep], k, v, False, 0.5)
    assert np.max(np.abs(o[keep] - o_ref)) < 1e-12 and np.max(np.abs(lse[keep] - lse_ref)) < 1e-12
    p, _, _ = A.softmax_rows((q[keep] @ k.T) * 0.5)
    dq, dk, dv = BS.backward_head_masked(q, k, v, do, a, 0.5)
    assert np.all(dq[8:16] == 0)
    dp = do[keep] @ v.T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    assert np.max(np.abs(dk - 0.5 * ds.T @ q[keep])) < 1e-12
    assert np.max(np.abs(dv - p.T @ do[keep])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    # Brute force: central differences of L = sum(dO * O) w.r.t. every input.
    n, d, blk, scale, h = 7, 3, 2, 0.8, 1e-6
    q, k, v, do = _qkvdo(n, d, 6 + causal)
    bm = np.array([[1, 0, 1, 1], [0, 1, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1]])
    a = BS.allowed_mask(n, bm, blk, causal)
    assert a.any(axis=1).all()

    def loss(q_, k_, v_):
        return float(np.sum(do * BS.forward_head_masked(q_, k_, v_, a, scale)[0]))

    grads = BS.backward_head_masked(q, k, v, do, a, scale)
    for which, g in enumerate(grads):
        args = [q, k, v]
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.max(np.abs(num - g)) < 1e-7, (which, np.max(np.abs(num - g)))


def test_batched_forms_and_mask_shapes():
    b_, h_, n, d, blk = 2, 3, 20, 4, 8
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((b_, h_, n, d)) for _ in range(4))
    nb = 3
    per_head = rng.integers(0, 2, size=(b_, h_, nb, nb))
    per_head[..., np.arange(nb), np.arange(nb)] = 1
    o, lse = BS.forward_blocksparse(q, k, v, per_head, False, None, blk)
    g = BS.backward_blocksparse(q, k, v, do, per_head, False, None, blk)
    for b in range(b_):
        for h in range(h_):
            a = BS.allowed_mask(n, per_head[b, h], blk, False)
            o1, lse1 = BS.forward_head_masked(q[b, h], k[b, h], v[b, h], a, 1 / np.sqrt(d))
            assert np.max(np.abs(o[b, h] - o1)) < 1e-14 and np.max(np.abs(lse[b, h] - lse1)) < 1e-14
    shared = per_head[0, 0]
    o2, _ = BS.forward_blocksparse(q, k, v, shared, True, 0.25, blk)
    o3, _ = BS.forward_blocksparse(q, k, v, np.broadcast_to(shared, (b_, h_, nb, nb)), True, 0.25, blk)
    assert np.array_equal(o2, o3)
    assert all(x.shape == q.shape for x in g)
