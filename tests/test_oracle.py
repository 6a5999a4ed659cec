"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: values the pages
print for their worked examples (``tests/golden/``), closed forms, invariants
the pages state, special cases, central finite differences, and the float64
CPU ``scaled_dot_product_attention`` of PyTorch with its autograd.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import online as OL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------


def test_paper_notes_worked_example_printed_values():
    g = _load("paper_notes_worked_example.json")
    tol = 0.5 * 10 ** (-g["printed_decimals"]) + 1e-12
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V"))
    s = A.scores(q, k, g["scale"], g["causal"])
    np.testing.assert_array_equal(s, np.array(g["S"], dtype=np.float64))
    p, m, l = A.softmax_rows(s)
    np.testing.assert_array_equal(m, np.array(g["row_max"], dtype=np.float64))
    np.testing.assert_allclose(l, g["row_l"], atol=tol, rtol=0)
    np.testing.assert_allclose(np.exp(s - m[:, None]), g["row_f"], atol=tol, rtol=0)
    np.testing.assert_allclose(p, g["P"], atol=tol, rtol=0)
    o, lse = A.forward_head(q, k, v, causal=False, scale=g["scale"])
    np.testing.assert_allclose(o, g["O"], atol=tol, rtol=0)


def test_paper_notes_worked_example_closed_form():
    # Row scores [1, 3] and [2, 4]: P = [1/(1+e^2), e^2/(1+e^2)], LSE = max + ln(1 + e^-2).
    q = np.eye(2)
    k = np.array([[1.0, 2.0], [3.0, 4.0]])
    v = np.eye(2)
    o, lse = A.forward_head(q, k, v, scale=1.0)
    p0 = 1.0 / (1.0 + math.e**2)
    np.testing.assert_allclose(o, [[p0, 1 - p0], [p0, 1 - p0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, [3 + math.log1p(math.exp(-2)), 4 + math.log1p(math.exp(-2))], rtol=0, atol=1e-15)


def test_aicassindra_tiny_example_running_stats():
    g = _load("aicassindra_tiny_example.json")
    tol = 0.5 * 10 ** (-g["printed_decimals"]) + 1e-12
    trace = OL.online_trace(g["blocks"])
    (m_a, l_a, r_a), (m_b, l_b, r_b) = trace
    assert m_a == g["after_block_A"]["m"] and r_a == 1.0
    assert abs(l_a - g["after_block_A"]["l"]) <= tol
    assert abs(r_b - g["rescale_when_B_arrives"]) <= tol
    blk_b = np.array(g["blocks"][1], dtype=np.float64)
    assert abs(np.exp(blk_b - m_b).sum() - g["block_B_terms"]) <= tol
    assert m_b == g["after_block_B"]["m"]
    assert abs(l_b - g["after_block_B"]["l"]) <= tol
    # One-shot over the whole row through the oracle: q = [1], keys = the scores.
    scores = np.concatenate([np.array(b, dtype=np.float64) for b in g["blocks"]])
    q = np.ones((1, 1))
    k = scores[:, None]
    v = np.eye(4)
    o, lse = A.forward_head(q, k, v, scale=1.0)
    assert abs(math.exp(lse[0] - scores.max()) - g["one_shot_l"]) <= tol
    # Streaming and one-shot agree far beyond the printed digits.
    assert abs((m_b + math.log(l_b)) - lse[0]) <= 1e-14
    np.testing.assert_allclose(o[0], np.exp(scores - lse[0]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Invariants the pages state, and special cases with closed forms
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k = _rand(1, 37, 8), _rand(2, 37, 8)
    p, _, _ = A.softmax_rows(A.scores(q, k, 0.7, causal))
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)


def test_shift_invariance_of_scores():
    # Adding u to every key adds scale*q_i.u to row i of S: O is unchanged,
    # LSE_i moves by exactly that constant.
    n, d, scale = 29, 6, 0.4
    q, k, v = _rand(3, n, d), _rand(4, n, d), _rand(5, n, d)
    u = _rand(6, d)
    for causal in (False, True):
        o1, l1 = A.forward_head(q, k, v, causal, scale)
        o2, l2 = A.forward_head(q, k + u[None, :], v, causal, scale)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, scale * (q @ u), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 5, 64, 77, 130])
def test_tiled_online_softmax_equals_one_shot(causal, n):
    d = 5
    q, k, v = _rand(10 + n, n, d), _rand(20 + n, n, d), _rand(30 + n, n, d)
    o_ref, l_ref = A.forward_head(q, k, v, causal, 0.9)
    for bq, bk in [(1, 1), (2, 3), (3, 2), (7, 7), (64, 64), (128, 128), (n, n), (5, 64), (64, 5)]:
        o, lse = OL.flash_forward_head(q, k, v, causal, 0.9, bq, bk)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_merge_rule_over_uneven_partitions_and_any_grouping(causal):
    """The two-block merge rule ("Tiling: Block-by-Block Softmax") folded over
    random uneven cuts of the keys, left to right or as a balanced tree, gives
    the one-shot softmax (the merge is associative)."""
    n, d = 97, 6
    q, k, v = _rand(61, n, d), _rand(62, n, d), _rand(63, n, d)
    o_ref, l_ref = A.forward_head(q, k, v, causal, 0.7)
    rng = np.random.default_rng(64)
    for trial in range(6):
        cuts = np.sort(rng.choice(np.arange(1, n), size=int(rng.integers(1, 12)), replace=False))
        for tree in (False, True):
            o, lse = OL.flash_forward_head(q, k, v, causal, 0.7, block_q=int(rng.integers(1, 40)), key_bounds=cuts,
                                           tree=tree)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)


def test_single_key_and_first_causal_row():
    q, k, v = _rand(7, 1, 4), _rand(8, 1, 4), _rand(9, 1, 4)
    o, lse = A.forward_head(q, k, v, False, 0.3)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q @ k.T)[0], rtol=0, atol=1e-15)
    q, k, v = _rand(7, 9, 4), _rand(8, 9, 4), _rand(9, 9, 4)
    o, lse = A.forward_head(q, k, v, True, 0.3)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - 0.3 * q[0] @ k[0]) <= 1e-15


def test_zero_queries_give_uniform_weights():
    n, d = 13, 3
    q = np.zeros((n, d))
    k, v = _rand(11, n, d), _rand(12, n, d)
    o, lse = A.forward_head(q, k, v, False, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), (n, d)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(n), rtol=0, atol=1e-14)
    o, lse = A.forward_head(q, k, v, True, 1.0)
    prefix = np.cumsum(v, 0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-14)


def test_linearity_in_values():
    n, d = 17, 4
    q, k = _rand(13, n, d), _rand(14, n, d)
    o, _ = A.forward_head(q, k, np.ones((n, d)), True, 0.5)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    v1, v2 = _rand(15, n, d), _rand(16, n, d)
    o1, _ = A.forward_head(q, k, v1, False, 0.5)
    o2, _ = A.forward_head(q, k, v2, False, 0.5)
    o3, _ = A.forward_head(q, k, 2.0 * v1 - 3.0 * v2, False, 0.5)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=0, atol=1e-13)


def test_joint_key_value_permutation():
    n, d = 21, 5
    q, k, v = _rand(17, n, d), _rand(18, n, d), _rand(19, n, d)
    perm = np.random.default_rng(20).permutation(n)
    o1, l1 = A.forward_head(q, k, v, False, 0.6)
    o2, l2 = A.forward_head(q, k[perm], v[perm], False, 0.6)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_paper_notes_pseudocode_step4_does_not_reproduce_softmax():
    """The Paper Notes page's printed step 4 is read as a garble.

    Written out literally (each block divided by the running sum of that
    moment, the accumulator rescaled by the old-max factor only) it drifts
    away from the one-shot softmax; the oracle's tiled loop follows the other
    two pages instead.  This test documents the size of the disagreement.
    """
    n, d, blk = 8, 4, 2
    q, k, v = _rand(21, n, d), _rand(22, n, d), _rand(23, n, d)
    o_ref, _ = A.forward_head(q, k, v, False, 1.0)
    o_lit = np.zeros((n, d))
    for i in range(n):
        m_g, l_g, acc = -np.inf, 0.0, np.zeros(d)
        for j0 in range(0, n, blk):
            s = q[i] @ k[j0 : j0 + blk].T
            m_loc = s.max()
            f_loc = np.exp(s - m_loc)
            l_loc = f_loc.sum()
            m_new = max(m_g, m_loc)
            s_old = math.exp(m_g - m_new) if np.isfinite(m_g) else 0.0
            s_new = math.exp(m_loc - m_new)
            l_g = s_old * l_g + s_new * l_loc
            m_g = m_new
            acc = s_old * acc + (s_new * f_loc / l_g) @ v[j0 : j0 + blk]
        o_lit[i] = acc
    assert np.max(np.abs(o_lit - o_ref)) > 0.1
    o_fix, _ = OL.flash_forward_head(q, k, v, False, 1.0, 1, blk)
    np.testing.assert_allclose(o_fix, o_ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# A library routine: PyTorch's float64 CPU attention and its autograd
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 3), (19, 8), (70, 16)])
def test_forward_and_gradients_match_torch_cpu_float64(causal, n, d):
    b, h = 2, 3
    rng = np.random.default_rng(100 + n + d)
    q, k, v, do = (rng.standard_normal((b, h, n, d)) for _ in range(4))
    o, _ = A.forward(q, k, v, causal)  # default scale 1/sqrt(d)
    dq, dk, dv = A.backward(q, k, v, do, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    # An explicit scale other than the default.
    o2, _ = A.forward(q, k, v, causal, scale=0.37)
    to2 = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=causal, scale=0.37
    )
    np.testing.assert_allclose(o2, to2.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Gradients: finite differences and identities
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (3, 2), (6, 4), (8, 3)])
def test_gradients_by_central_finite_differences(causal, n, d):
    rng = np.random.default_rng(200 + 10 * n + d + causal)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.8
    dq, dk, dv = A.backward_head(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        o, _ = A.forward_head(qq, kk, vv, causal, scale)
        return float(np.sum(do * o))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(n, d):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7, (which, idx, fd, grad[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    n, d, scale = 33, 7, 0.45
    rng = np.random.default_rng(300 + causal)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = A.backward_head(q, k, v, do, causal, scale)
    o, _ = A.forward_head(q, k, v, causal, scale)
    # Shifting every key by one vector leaves O unchanged, so the key
    # gradients sum to zero.
    np.testing.assert_allclose(dk.sum(0), 0.0, rtol=0, atol=1e-12)
    # Rows of P sum to one, so the value gradients sum to the output gradients.
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=0, atol=1e-12)
    # S is bilinear in Q and K: <dQ, Q> = <dK, K> = <dS, S>/1.
    assert abs(np.sum(dq * q) - np.sum(dk * k)) <= 1e-12
    # sum_j P_ij dP_ij = sum_k dO_ik O_ik.
    lse, dsum = A.head_row_stats(q, k, v, do, causal, scale, chunk=5)
    np.testing.assert_allclose(dsum, np.sum(do * o, -1), rtol=0, atol=1e-12)
    if causal:
        # Query 0 sees only key 0, where P = 1: its score gradient vanishes.
        np.testing.assert_array_equal(dq[0], 0.0)


# ---------------------------------------------------------------------------
# Row-restricted helpers used at long sequence lengths
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("causal", [False, True])
def test_row_helpers_agree_with_whole_head(causal):
    n, d, scale = 53, 6, 0.5
    rng = np.random.default_rng(400 + causal)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, lse = A.forward_head(q, k, v, causal, scale)
    dq, dk, dv = A.backward_head(q, k, v, do, causal, scale)
    rows = np.array([0, 1, 7, 26, 51, 52])
    o_r, lse_r = A.forward_rows(q, k, v, rows, causal, scale)
    np.testing.assert_allclose(o_r, o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_r, lse[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(A.backward_query_rows(q, k, v, do, rows, causal, scale), dq[rows], rtol=0, atol=1e-13)
    lse_all, dsum_all = A.head_row_stats(q, k, v, do, causal, scale, chunk=7)
    np.testing.assert_allclose(lse_all, lse, rtol=0, atol=1e-13)
    dk_r, dv_r = A.backward_key_rows(q, k, v, do, rows, lse_all, dsum_all, causal, scale, chunk=11)
    np.testing.assert_allclose(dk_r, dk[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv_r, dv[rows], rtol=0, atol=1e-13)
