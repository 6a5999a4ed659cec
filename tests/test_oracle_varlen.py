"""Pins of the unequal-length oracle and of the split-K/V merge
(oracle/varlen.py).

Rows of a softmax are independent, so attention of Nq queries over Nk keys is
a subset of the rows of a square problem: the pins embed each case in a square
one and compare with the dense oracle (pinned in test_oracle.py).  The merge
is pinned against the one-shot definition over many split points, and against
the values the pages print for their two-block example.
"""

import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import varlen as VL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _r(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_is_dense(causal):
    n, d = 23, 5
    q, k, v, do = (_r((n, d), s) for s in range(4))
    o, lse = VL.forward_qk(q, k, v, causal, 0.4)
    o_r, lse_r = A.forward_head(q, k, v, causal, 0.4)
    assert np.max(np.abs(o - o_r)) < 1e-12 and np.max(np.abs(lse - lse_r)) < 1e-12
    for x, y in zip(VL.backward_qk(q, k, v, do, causal, 0.4), A.backward_head(q, k, v, do, causal, 0.4)):
        assert np.max(np.abs(x - y)) < 1e-12


@pytest.mark.parametrize("nq", [1, 5, 16])
def test_causal_bottom_right_is_the_last_rows_of_a_square_problem(nq):
    # Nq queries after Nk - Nq earlier tokens: the last Nq rows of the square
    # causal problem whose earlier rows are anything.
    nk, d = 19, 4
    q, k, v, do = _r((nq, d), 1), _r((nk, d), 2), _r((nk, d), 3), _r((nq, d), 4)
    qf = np.concatenate([_r((nk - nq, d), 5), q])
    dof = np.concatenate([np.zeros((nk - nq, d)), do])
    o, lse = VL.forward_qk(q, k, v, True, 0.7)
    o_r, lse_r = A.forward_head(qf, k, v, True, 0.7)
    assert np.max(np.abs(o - o_r[nk - nq:])) < 1e-12 and np.max(np.abs(lse - lse_r[nk - nq:])) < 1e-12
    # Gradients: the earlier rows carry dO = 0, so they add nothing to dK, dV.
    dq, dk, dv = VL.backward_qk(q, k, v, do, True, 0.7)
    dq_r, dk_r, dv_r = A.backward_head(qf, k, v, dof, True, 0.7)
    assert np.max(np.abs(dq - dq_r[nk - nq:])) < 1e-12
    assert np.max(np.abs(dk - dk_r)) < 1e-12 and np.max(np.abs(dv - dv_r)) < 1e-12


def test_more_queries_than_keys_causal():
    # Nq > Nk: the first Nq - Nk rows see no key; the rest form the square
    # causal problem on the last Nk rows.
    nq, nk, d = 12, 7, 3
    q, k, v, do = _r((nq, d), 6), _r((nk, d), 7), _r((nk, d), 8), _r((nq, d), 9)
    o, lse = VL.forward_qk(q, k, v, True, 0.5)
    assert np.all(o[: nq - nk] == 0) and np.all(np.isneginf(lse[: nq - nk]))
    o_r, lse_r = A.forward_head(q[nq - nk:], k, v, True, 0.5)
    assert np.max(np.abs(o[nq - nk:] - o_r)) < 1e-12 and np.max(np.abs(lse[nq - nk:] - lse_r)) < 1e-12
    dq, dk, dv = VL.backward_qk(q, k, v, do, True, 0.5)
    assert np.all(dq[: nq - nk] == 0)
    g = A.backward_head(q[nq - nk:], k, v, do[nq - nk:], True, 0.5)
    assert np.max(np.abs(dq[nq - nk:] - g[0])) < 1e-12
    assert np.max(np.abs(dk - g[1])) < 1e-12 and np.max(np.abs(dv - g[2])) < 1e-12


@pytest.mark.parametrize("nq,nk", [(3, 17), (17, 3)])
def test_non_causal_rows_match_square_problems(nq, nk):
    d = 4
    q, k, v = _r((nq, d), 10), _r((nk, d), 11), _r((nk, d), 12)
    o, lse = VL.forward_qk(q, k, v, False, 0.6)
    # Embed the queries, in chunks of at most Nk rows, into square problems.
    for s0 in range(0, nq, nk):
        qq = q[s0: s0 + nk]
        pad = np.concatenate([qq, np.zeros((nk - len(qq), d))])
        o_r, lse_r = A.forward_head(pad, k, v, False, 0.6)
        assert np.max(np.abs(o[s0: s0 + nk] - o_r[: len(qq)])) < 1e-12
        assert np.max(np.abs(lse[s0: s0 + nk] - lse_r[: len(qq)])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(10,), (1, 2, 3), (5, 6, 30), (0, 40)])
def test_split_merge_equals_one_shot(cuts, causal):
    nq, nk, d = 9, 40, 5
    q, k, v = _r((nq, d), 13), _r((nk, d), 14), _r((nk, d), 15)
    a = VL.allowed_qk(nq, nk, causal)
    edges = [0] + [c for c in cuts if 0 < c < nk] + [nk]
    stats = None
    for lo, hi in zip(edges[:-1], edges[1:]):
        p = VL.partial_stats(q, k[lo:hi], v[lo:hi], 0.3, a[:, lo:hi])
        stats = p if stats is None else VL.merge_two(stats, p)
    o, lse = VL.finish(stats)
    o_r, lse_r = VL.forward_qk(q, k, v, causal, 0.3)
    assert np.max(np.abs(o - o_r)) < 1e-12 and np.max(np.abs(lse - lse_r)) < 1e-12


def test_merge_reproduces_the_pages_two_block_example():
    # aicassindra, "A tiny worked example": scores [1, 3] then [2, 5] (scale
    # 1, one query); the page prints l = 1.135 after block A and 1.203 after B.
    g = json.load(open(os.path.join(GOLDEN, "aicassindra_tiny_example.json")))
    q = np.array([[1.0]])
    blocks = [np.array(b, dtype=np.float64)[:, None] for b in g["blocks"]]
    ones = [np.ones((1, len(b)), dtype=bool) for b in g["blocks"]]
    v = [np.eye(4)[:2], np.eye(4)[2:]]
    p_a = VL.partial_stats(q, blocks[0], v[0], 1.0, ones[0])
    assert p_a[0][0] == g["after_block_A"]["m"] and round(p_a[1][0], 3) == g["after_block_A"]["l"]
    m, l, acc = VL.merge_two(p_a, VL.partial_stats(q, blocks[1], v[1], 1.0, ones[1]))
    assert m[0] == g["after_block_B"]["m"] and round(l[0], 3) == g["after_block_B"]["l"]
    o, _ = VL.finish((m, l, acc))
    s = np.array([1.0, 3.0, 2.0, 5.0])
    assert np.max(np.abs(o[0] - np.exp(s) / np.exp(s).sum())) < 1e-15


def test_batched_forms():
    b_, h_, nq, nk, d = 2, 2, 5, 11, 4
    rng = np.random.default_rng(16)
    q, do = rng.standard_normal((b_, h_, nq, d)), rng.standard_normal((b_, h_, nq, d))
    k, v = rng.standard_normal((b_, h_, nk, d)), rng.standard_normal((b_, h_, nk, d))
    o, lse = VL.forward_qk_batched(q, k, v, True)
    g = VL.backward_qk_batched(q, k, v, do, True)
    for b in range(b_):
        for h in range(h_):
            o1, lse1 = VL.forward_qk(q[b, h], k[b, h], v[b, h], True, 1 / np.sqrt(d))
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], lse1)
    assert g[0].shape == q.shape and g[1].shape == k.shape
