"""Invariants of exact attention checked on the GPU outputs themselves (no
oracle), through the C ABI, bf16.

* Shift invariance (Paper Notes, "What Are We Computing?": softmax of each
  score row): adding the same vector u to every key adds scale * q_i . u to
  every score of row i, so O is unchanged and LSE_i grows by scale * q_i . u.
  Inputs are small multiples of 1/8, so K + u is exact in bf16 and the shift
  of each row is exact.
* Joint permutation of the key and value rows (no mask): O and LSE are
  unchanged, dK and dV are permuted alike, dQ is unchanged.
* The key gradients of a head sum to zero: the score row's softmax makes
  sum_j dS_ij = 0, so sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0.
Tolerances: the bf16 rule for tensors (max abs 2e-2, relative Frobenius
1e-2); sums against the norm of the summed tensor.
"""

import math

import numpy as np
import pytest
import torch

from tests.gpu_util import BF16_REL_FRO, assert_close, download

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


def _eighths(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64) / 8.0


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 2, 300, 64), (1, 2, 257, 128)])
def test_shift_of_every_key_by_one_vector(shape, causal):
    E = _api()
    b, h, n, d = shape
    _announce("shift invariance", shape, causal)
    rng = np.random.default_rng(11 + n + d)
    q = _eighths(rng, shape, -2, 2)
    k = _eighths(rng, shape, -4, 4)
    v = rng.standard_normal(shape)
    u = _eighths(rng, (b, h, 1, d), -2, 2)
    scale = 1.0 / math.sqrt(d)
    qg, vg = _bf16(q), _bf16(v)
    o1, l1 = E.attn_fwd(qg, _bf16(k), vg, causal=causal, scale=scale)
    o2, l2 = E.attn_fwd(qg, _bf16(k + u), vg, causal=causal, scale=scale)
    torch.cuda.synchronize()
    shift = scale * np.einsum("bhnd,bhd->bhn", q, u[:, :, 0, :])
    assert_close(download(o2), download(o1), "bf16", "O after the shift")
    err = float(np.max(np.abs(download(l2) - download(l1) - shift)))
    assert err <= 2e-4, f"LSE shift: max error {err:.3e}"


@pytest.mark.parametrize("shape", [(2, 2, 300, 64), (1, 2, 257, 128)])
def test_joint_permutation_of_keys_and_values(shape):
    E = _api()
    b, h, n, d = shape
    _announce("permutation", shape)
    rng = np.random.default_rng(21 + n + d)
    q, k, v, do = (rng.standard_normal(shape) for _ in range(4))
    perm = rng.permutation(n)
    scale = 1.0 / math.sqrt(d)
    qg, dog = _bf16(q), _bf16(do)
    o1, l1 = E.attn_fwd(qg, _bf16(k), _bf16(v), causal=False, scale=scale)
    g1 = E.attn_bwd(qg, _bf16(k), _bf16(v), o1, dog, l1, causal=False, scale=scale)
    kp, vp = k[:, :, perm], v[:, :, perm]
    o2, l2 = E.attn_fwd(qg, _bf16(kp), _bf16(vp), causal=False, scale=scale)
    g2 = E.attn_bwd(qg, _bf16(kp), _bf16(vp), o2, dog, l2, causal=False, scale=scale)
    torch.cuda.synchronize()
    assert_close(download(o2), download(o1), "bf16", "O")
    assert float(np.max(np.abs(download(l2) - download(l1)))) <= 1e-4
    assert_close(download(g2[0]), download(g1[0]), "bf16", "dQ")
    assert_close(download(g2[1]), download(g1[1])[:, :, perm], "bf16", "dK (permuted)")
    assert_close(download(g2[2]), download(g1[2])[:, :, perm], "bf16", "dV (permuted)")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 2, 300, 64), (1, 2, 1000, 128)])
def test_key_gradients_of_a_head_sum_to_zero(shape, causal):
    E = _api()
    b, h, n, d = shape
    _announce("sum of dK", shape, causal)
    rng = np.random.default_rng(31 + n + d)
    q, k, v, do = (_bf16(rng.standard_normal(shape)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd(q, k, v, causal=causal, scale=scale)
    _, dk, _ = E.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    dkh = download(dk).reshape(b * h, n, d)
    total = dkh.sum(axis=1)  # [heads, d]
    # Each row's rounding (bf16 output) is independent: the sum's error grows
    # like sqrt(n) times one row's; compare with the head's Frobenius norm.
    rel = float(np.linalg.norm(total) / np.linalg.norm(dkh))
    assert rel <= BF16_REL_FRO, f"|sum_j dK_j| / ||dK||_F = {rel:.3e}"
