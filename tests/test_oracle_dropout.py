"""Pins of the dropout oracle (oracle/dropout.py).

The attention part is pinned against the plain oracle (no dropout), finite
differences with the mask held fixed, an element-by-element route through
the saved LSE, and the row identity behind D.  The generator is pinned by
what a counter-based generator must satisfy: a bijection of the counter for a
fixed key (no collisions), output bits that are uniform and that change by
about half when one counter bit flips, keep rates within binomial bounds, and
masks that change with the seed and the offset.  Its identity with
Philox4x32-10 is pinned by the published known-answer vectors
(tests/golden/philox4x32_10_kat.json): a wrong multiplier, key increment,
round count or word order fails them.
"""

import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import dropout as DR


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answer_vectors():
    """The generator reproduces the published Philox4x32-10 known answers
    (Salmon et al., SC 2011; the Random123 known-answer file): all-zero and
    all-ones counters and keys, and the pi-digit counter and key."""
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    assert len(kat["vectors"]) == 3
    for vec in kat["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        got = DR.philox4x32_10(*c, *k)
        assert [int(np.asarray(w)) for w in got] == [int(x, 16) for x in vec["expected"]], vec


def test_philox_known_answer_fails_a_planted_mistake(monkeypatch):
    """The known answers catch a wrong constant: a planted change of the
    second key increment (in the oracle, on the CPU) no longer reproduces the
    pi-digit vector."""
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        vec = json.load(f)["vectors"][2]
    c = [int(x, 16) for x in vec["counter"]]
    k = [int(x, 16) for x in vec["key"]]
    monkeypatch.setattr(DR, "_W1", DR._W1 ^ 1)
    got = DR.philox4x32_10(*c, *k)
    assert [int(np.asarray(w)) for w in got] != [int(x, 16) for x in vec["expected"]]


def _r(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_the_plain_definition(causal):
    n, d = 21, 6
    q, k, v, do = (_r((n, d), s) for s in range(4))
    z = DR.keep_mask(0, n, n, 0.0, 99)
    assert z.all()
    o, lse = DR.forward_head(q, k, v, causal, 0.3, z, 0.0)
    o_r, lse_r = A.forward_head(q, k, v, causal, 0.3)
    assert np.max(np.abs(o - o_r)) < 1e-12 and np.max(np.abs(lse - lse_r)) < 1e-12
    for x, y in zip(DR.backward_head(q, k, v, do, causal, 0.3, z, 0.0), A.backward_head(q, k, v, do, causal, 0.3)):
        assert np.max(np.abs(x - y)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    n, d, p, scale = 6, 3, 0.3, 0.7
    q, k, v, do = (_r((n, d), 10 + s) for s in range(4))
    z = np.random.default_rng(5).random((n, n)) >= p
    g = DR.backward_head(q, k, v, do, causal, scale, z, p)

    def loss(qq, kk, vv):
        return float(np.sum(DR.forward_head(qq, kk, vv, causal, scale, z, p)[0] * do))

    h = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(num - g[which])) < 1e-7


def test_element_by_element_through_lse():
    # O_i = sum_j z_ij exp(S_ij - LSE_i) V_j / (1 - p), one element at a time.
    n, d, p, scale = 9, 4, 0.25, 0.5
    q, k, v = (_r((n, d), 20 + s) for s in range(3))
    z = DR.keep_mask(2, n, n, p, 4242, 3)
    o, lse = DR.forward_head(q, k, v, True, scale, z, p)
    s = 1.0 / (1.0 - float(np.float32(p)))
    for i in range(n):
        acc = np.zeros(d)
        for j in range(i + 1):
            if z[i, j]:
                acc += np.exp(float(q[i] @ k[j]) * scale - lse[i]) * v[j]
        assert np.max(np.abs(acc * s - o[i])) < 1e-12


def test_row_term_identity_holds_with_dropout():
    n, d, p = 12, 5, 0.4
    q, k, v, do = (_r((n, d), 30 + s) for s in range(4))
    z = DR.keep_mask(1, n, n, p, 7)
    P, _ = DR._probs(q, k, False, 0.6)
    o, _ = DR.forward_head(q, k, v, False, 0.6, z, p)
    s = 1.0 / (1.0 - float(np.float32(p)))
    dp = (do @ v.T) * z * s
    assert np.max(np.abs((P * dp).sum(-1) - (do * o).sum(-1))) < 1e-12


def test_threshold():
    assert DR.threshold(0.0) == 0
    assert DR.threshold(0.5) == 2**31
    assert DR.threshold(0.25) == 2**30
    assert DR.threshold(np.nextafter(np.float32(1), np.float32(0))) == 2**32 - 256
    assert DR.threshold(1.0) == 2**32 - 1


def test_generator_is_a_bijection_of_the_counter():
    c = np.arange(1 << 16, dtype=np.uint64)
    w = DR.philox4x32_10(c, c * np.uint64(3), np.uint64(5), np.uint64(0), 1234, 5678)
    packed = {(int(a), int(b), int(x), int(y)) for a, b, x, y in zip(*w)}
    assert len(packed) == 1 << 16


def test_generator_output_bits_are_uniform():
    c = np.arange(1 << 15, dtype=np.uint64)
    words = np.concatenate(DR.philox4x32_10(c, 0, 0, 0, 42, 0))
    bits = ((words[:, None] >> np.arange(32, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.float64)
    frac = bits.mean(axis=0)  # each bit is set half the time
    assert np.all(np.abs(frac - 0.5) < 5 * 0.5 / np.sqrt(len(words)))
    hist = np.bincount((words >> np.uint64(28)).astype(np.int64), minlength=16)  # top nibble
    exp = len(words) / 16
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    assert chi2 < 45.0  # 15 degrees of freedom: p < 1e-4


def test_one_counter_bit_flips_about_half_the_output():
    rng = np.random.default_rng(3)
    base = rng.integers(0, 2**32, size=(4, 2000), dtype=np.uint64)
    w0 = np.stack(DR.philox4x32_10(*base, 11, 22))
    for word in range(4):
        for bit in (0, 13, 31):
            flipped = base.copy()
            flipped[word] ^= np.uint64(1 << bit)
            w1 = np.stack(DR.philox4x32_10(*flipped, 11, 22))
            x = w0 ^ w1
            ones = sum(int(bin(int(v)).count("1")) for v in x.ravel())
            frac = ones / (x.size * 32)
            assert abs(frac - 0.5) < 0.01


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate(p):
    z = DR.keep_mask(0, 300, 300, p, 2024, 0)
    nobs = z.size
    sd = np.sqrt(p * (1 - p) / nobs)
    assert abs(z.mean() - (1 - p)) < 6 * sd


def test_masks_change_with_head_seed_and_offset():
    a = DR.keep_mask(0, 128, 128, 0.5, 1, 0)
    for other in (DR.keep_mask(1, 128, 128, 0.5, 1, 0), DR.keep_mask(0, 128, 128, 0.5, 2, 0),
                  DR.keep_mask(0, 128, 128, 0.5, 1 << 33, 0), DR.keep_mask(0, 128, 128, 0.5, 1, 1)):
        agree = (a == other).mean()
        assert abs(agree - 0.5) < 0.02  # independent masks agree half the time
    assert np.array_equal(a, DR.keep_mask(0, 128, 128, 0.5, 1, 0))


def test_batched_forms():
    shape = (2, 2, 10, 4)
    q, k, v, do = (_r(shape, 40 + s) for s in range(4))
    o, lse = DR.forward(q, k, v, True, 0.5, 0.2, 77, 5)
    g = DR.backward(q, k, v, do, True, 0.5, 0.2, 77, 5)
    for b in range(2):
        for h in range(2):
            z = DR.keep_mask(b * 2 + h, 10, 10, 0.2, 77, 5)
            o1, l1 = DR.forward_head(q[b, h], k[b, h], v[b, h], True, 0.5, z, 0.2)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)
    assert g[0].shape == shape
