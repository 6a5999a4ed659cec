"""GPU parity of attention under a key padding mask (attn_fwd_kpad /
attn_bwd_kpad) through the C ABI, against the float64 oracle of
oracle/keypad.py.

Key lengths cover the edges of the 64-key tiles and 128-key blocks (1, 63,
64, 65, 127, 128, 129), a batch with no key at all, lengths outside [0, N]
(clamped), and N itself.  The padded rows of K and V are filled with large
finite values, which must not reach any output.

A batch with one valid key sends every row's whole probability to that key,
so its dV row is the sum of all N rows of dO (magnitude ~sqrt(N) per entry,
up to ~40 here), where the output's own bf16 rounding alone (2^-9 relative)
exceeds the absolute bound of the other tests.  The gradients are therefore
held elementwise to |gpu - oracle| <= 2e-2 + 2^-7 |oracle| (four times that
rounding on top of the usual bound) and to the usual relative Frobenius
bound; fp32 to 1e-5 + 1e-6 |oracle|.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import keypad as KP
from tests.gpu_util import BF16_MAX_ABS, BF16_REL_FRO, F32_MAX_ABS, assert_close, download, errors, upload

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


def _inputs(seed, shape, dtype, lens):
    inp = synth.qkvdo(seed, shape, dtype)
    rng = np.random.default_rng(seed + 1)
    N = shape[2]
    for name in ("k", "v"):
        raw = inp[name + "_raw"].copy()
        for b, L in enumerate(lens):
            L = KP.clamp_len(L, N)
            junk = (300.0 * rng.standard_normal((shape[1], N - L, shape[3]))).astype(np.float32)
            if dtype == "bf16":
                raw[b, :, L:] = synth.f32_to_bf16_bits(junk)
            else:
                raw[b, :, L:] = junk
        inp[name + "_raw"] = raw
        inp[name] = (synth.bf16_bits_to_f32(raw) if dtype == "bf16" else raw).astype(np.float64)
    return inp


def _close_rel(got, ref, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    excess = np.abs(got - ref) - (2.0 ** -7 if dtype == "bf16" else 1e-6) * np.abs(ref)
    bound = BF16_MAX_ABS if dtype == "bf16" else F32_MAX_ABS
    assert np.max(excess) <= bound, f"{what}: error beyond {bound} + rel: {np.max(excess):.3e}"
    if dtype == "bf16":
        _, rel = errors(got, ref)
        assert rel <= BF16_REL_FRO, f"{what}: rel Frobenius {rel:.3e}"


def _compare_lse(got, ref, dtype):
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "rows without keys: LSE must be -inf exactly there"
    if np.any(~empty):
        assert_close(got[~empty], ref[~empty], dtype, "LSE")


CASES = [
    ((3, 2, 129, 64), [0, 65, 129]),
    ((4, 2, 200, 128), [1, 63, 64, 200]),
    ((3, 1, 300, 128), [127, 128, 129]),
    ((2, 3, 256, 64), [-4, 1000]),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_key_padding_forward_backward(case, causal, dtype):
    shape, lens = case
    B, H, N, d = shape
    seed = 700 + N + d + 3 * causal
    _announce("kpad", shape, lens, dtype, "causal" if causal else "full", "seed", seed)
    E = _api()
    inp = _inputs(seed, shape, dtype, lens)
    q, k, v, do = (upload(inp[x + "_raw"], dtype) for x in ("q", "k", "v", "do"))
    key_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd_kpad(q, k, v, key_len, causal=causal, scale=scale)
    dq, dk, dv = E.attn_bwd_kpad(q, k, v, o, do, lse, key_len, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = KP.forward_keypad(inp["q"], inp["k"], inp["v"], lens, causal, scale)
    g_r = KP.backward_keypad(inp["q"], inp["k"], inp["v"], inp["do"], lens, causal, scale)
    assert_close(download(o), o_r, dtype, "O")
    _compare_lse(download(lse), lse_r, dtype)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
        _close_rel(download(got), ref, dtype, name)
    # Padded keys: exactly zero gradients.
    dkh, dvh = download(dk), download(dv)
    for b, L in enumerate(lens):
        L = KP.clamp_len(L, N)
        assert np.all(dkh[b, :, L:] == 0) and np.all(dvh[b, :, L:] == 0)


def test_full_length_equals_plain_entry_points():
    """key_len = N everywhere gives attn_fwd / attn_bwd's results bit for bit
    (the same kernels, no key masked)."""
    shape = (2, 2, 333, 128)
    _announce("kpad full length", shape)
    E = _api()
    inp = synth.qkvdo(81, shape, "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    key_len = torch.full((2,), 333, dtype=torch.int32, device="cuda")
    for causal in (False, True):
        o1, l1 = E.attn_fwd(q, k, v, causal=causal)
        g1 = E.attn_bwd(q, k, v, o1, do, l1, causal=causal)
        o2, l2 = E.attn_fwd_kpad(q, k, v, key_len, causal=causal)
        g2 = E.attn_bwd_kpad(q, k, v, o2, do, l2, key_len, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


def test_key_padding_at_full_size():
    """N = 4096, d = 128 (the forward's 256-row and the dK/dV kernel's 128-key
    blocks, many of them wholly padded), every element against the oracle
    (run per batch on the host cores)."""
    from tests.gpu_util import oracle_map

    shape, lens = (2, 1, 4096, 128), [2049, 1000]
    E = _api()
    scale = 1.0 / math.sqrt(128)
    for causal in (False, True):
        _announce("kpad full size", shape, lens, "causal" if causal else "full")
        inp = _inputs(4343 + causal, shape, "bf16", lens)
        q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
        key_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o, lse = E.attn_fwd_kpad(q, k, v, key_len, causal=causal)
        dq, dk, dv = E.attn_bwd_kpad(q, k, v, o, do, lse, key_len, causal=causal)
        torch.cuda.synchronize()

        def ref(b):
            sl = {x: inp[x][b:b + 1] for x in ("q", "k", "v", "do")}
            fo = KP.forward_keypad(sl["q"], sl["k"], sl["v"], lens[b:b + 1], causal, scale)
            return fo, KP.backward_keypad(sl["q"], sl["k"], sl["v"], sl["do"], lens[b:b + 1], causal, scale)

        refs = oracle_map(ref, range(shape[0]))
        o_r = np.concatenate([r[0][0] for r in refs])
        lse_r = np.concatenate([r[0][1] for r in refs])
        g_r = [np.concatenate([r[1][i] for r in refs]) for i in range(3)]
        assert_close(download(o), o_r, "bf16", "O")
        _compare_lse(download(lse), lse_r, "bf16")
        for name, got, ref_g in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
            _close_rel(download(got), ref_g, "bf16", name)
