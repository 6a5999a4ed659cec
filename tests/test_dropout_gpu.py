"""GPU parity of attention with dropout (attn_fwd_dropout / attn_bwd_dropout)
through the C ABI, against the float64 oracle of oracle/dropout.py.

Two kinds of checks:
* the keep mask itself, bit for bit: inputs chosen so that an output entry is
  non-zero exactly when its element was kept (forward kernel, dK/dV kernel,
  dQ kernel separately);
* random inputs at the bf16 tolerance, with the oracle drawing the same mask.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import dropout as DR
from tests.gpu_util import BF16_MAX_ABS, BF16_REL_FRO, assert_close, download, errors, upload

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda().contiguous()


def _masks(B, H, n, p, seed, offset):
    return np.stack([DR.keep_mask(bh, n, n, p, seed, offset) for bh in range(B * H)]).reshape(B, H, n, n)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_mask_bit_for_bit(causal):
    # Q = 0: uniform probabilities over the visible keys; V = identity: O[i][j]
    # is the kept, rescaled probability of key j, zero when dropped.
    E = _api()
    B, H, n, d, p, seed, off = 2, 2, 128, 128, 0.3, 0x1234567890ABCDEF, 5
    _announce("dropout fwd mask", causal)
    q = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    k = _bf16(np.random.default_rng(1).standard_normal((B, H, n, d)))
    v = _bf16(np.broadcast_to(np.eye(n, d), (B, H, n, d)))
    o, _ = E.attn_fwd_dropout(q, k, v, p, seed, off, causal=causal)
    torch.cuda.synchronize()
    z = _masks(B, H, n, p, seed, off)
    if causal:
        z = z & np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(download(o) > 0, z)


@pytest.mark.parametrize("causal", [False, True])
def test_dkdv_kernel_mask_bit_for_bit(causal):
    # Q = 0, dO = identity: dV[j][i] is the kept, rescaled P_ij.
    E = _api()
    B, H, n, d, p, seed, off = 1, 3, 128, 128, 0.25, 77, 0
    _announce("dropout dkdv mask", causal)
    q = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    k = _bf16(np.random.default_rng(2).standard_normal((B, H, n, d)))
    v = _bf16(np.random.default_rng(3).standard_normal((B, H, n, d)))
    do = _bf16(np.broadcast_to(np.eye(n, d), (B, H, n, d)))
    o, lse = E.attn_fwd_dropout(q, k, v, p, seed, off, causal=causal)
    _, _, dv = E.attn_bwd_dropout(q, k, v, o, do, lse, p, seed, off, causal=causal)
    torch.cuda.synchronize()
    z = _masks(B, H, n, p, seed, off)
    if causal:
        z = z & np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(np.swapaxes(download(dv), -1, -2) > 0, z)


def test_dq_kernel_mask_bit_for_bit():
    # Q = 0, K = V = identity, dO = ones: dP_ij = Z_ij / (1 - p), so
    # dS_ij = (Z_ij / (1 - p) - D_i) / n, and dQ[i][j] = scale dS_ij > 0
    # exactly when Z_ij = 1 (D_i lies strictly between 0 and 1 / (1 - p)).
    E = _api()
    B, H, n, d, p, seed, off = 1, 2, 128, 128, 0.25, 2024, 9
    _announce("dropout dq mask")
    q = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    eye = _bf16(np.broadcast_to(np.eye(n, d), (B, H, n, d)))
    do = torch.ones((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    o, lse = E.attn_fwd_dropout(q, eye, eye, p, seed, off)
    dq, _, _ = E.attn_bwd_dropout(q, eye, eye, o, do, lse, p, seed, off)
    torch.cuda.synchronize()
    z = _masks(B, H, n, p, seed, off)
    assert not z.all(axis=-1).any() and z.any(axis=-1).all()
    assert np.array_equal(download(dq) > 0, z)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_p_zero_equals_the_plain_path(d, causal):
    # The forward does the plain path's arithmetic (kept probabilities times
    # 1.0): bit for bit.  The backward forms dP - D after the products rather
    # than in their accumulator, so it agrees to rounding.
    E = _api()
    shape = (2, 2, 333, d)
    _announce("dropout p=0 == plain", d, causal)
    inp = synth.qkvdo(8000 + d + causal, shape, "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    o1, l1 = E.attn_fwd_dropout(q, k, v, 0.0, 5, 0, causal=causal)
    o2, l2 = E.attn_fwd(q, k, v, causal=causal)
    g1 = E.attn_bwd_dropout(q, k, v, o2, do, l2, 0.0, 5, 0, causal=causal)
    g2 = E.attn_bwd(q, k, v, o2, do, l2, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), f"O: max diff {float((o1.float() - o2.float()).abs().max()):.3e}"
    assert torch.equal(l1, l2), f"LSE: max diff {float((l1 - l2).abs().max()):.3e}"
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        diff = float((a.float() - b.float()).abs().max())
        assert diff <= 4e-3, f"{name}: max diff {diff:.3e}"


CASES = [(2, 2, 200, 64), (1, 3, 257, 128), (1, 2, 64, 128)]


@pytest.mark.parametrize("p", [0.1, 0.3])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", CASES)
def test_random_inputs_match_the_oracle(shape, causal, p):
    E = _api()
    seed, off = 31337 + shape[2], 3
    _announce("dropout parity", shape, causal, p)
    inp = synth.qkvdo(8100 + shape[2] + shape[3], shape, "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(shape[3])
    o, lse = E.attn_fwd_dropout(q, k, v, p, seed, off, causal=causal, scale=scale)
    dq, dk, dv = E.attn_bwd_dropout(q, k, v, o, do, lse, p, seed, off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = DR.forward(inp["q"], inp["k"], inp["v"], causal, scale, p, seed, off)
    g_r = DR.backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, p, seed, off)
    assert_close(download(lse), lse_r, "bf16", "LSE")
    # Dropout scales outputs and gradients by 1 / (1 - p), and with them the
    # bf16 rounding of the results: the absolute bound scales alike (the
    # relative Frobenius bound is scale-free and stays 1e-2).
    s = 1.0 / (1.0 - p)
    for name, got, ref in (("O", o, o_r), ("dQ", dq, g_r[0]), ("dK", dk, g_r[1]), ("dV", dv, g_r[2])):
        g = download(got)
        assert np.all(np.isfinite(g)), name
        max_abs, rel = errors(g, ref)
        assert max_abs <= BF16_MAX_ABS * s, f"{name}: max abs {max_abs:.3e} > {BF16_MAX_ABS * s:.3e}"
        assert rel <= BF16_REL_FRO, f"{name}: rel Frobenius {rel:.3e}"


def test_seed_and_offset_select_different_masks():
    E = _api()
    B, H, n, d = 1, 1, 128, 128
    _announce("dropout seeds")
    q = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    k = _bf16(np.random.default_rng(4).standard_normal((B, H, n, d)))
    v = _bf16(np.broadcast_to(np.eye(n, d), (B, H, n, d)))
    outs = [download(E.attn_fwd_dropout(q, k, v, 0.5, s, o)[0]) > 0 for s, o in ((1, 0), (2, 0), (1, 1), (1, 0))]
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[3])
    for other in outs[1:3]:
        assert 0.4 < (outs[0] == other).mean() < 0.6
