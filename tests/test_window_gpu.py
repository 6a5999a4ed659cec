"""GPU parity of causal sliding-window attention (attn_fwd_window /
attn_bwd_window) through the C ABI, against the float64 oracle of
oracle/window.py.

Windows cover 1 (each row sees only itself), widths below, at and across the
64-key tile, the 128-key block and the 256-row forward / dQ workgroup, and
N - 1; a window of N or more must give the plain causal results bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import window as WO
from tests.gpu_util import assert_close, download, upload

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


CASES = [
    ((2, 2, 300, 64), 1),
    ((2, 2, 300, 64), 31),
    ((1, 3, 513, 128), 64),
    ((1, 3, 513, 128), 100),
    ((2, 1, 700, 64), 129),
    ((2, 2, 1024, 128), 256),
    ((1, 2, 1024, 128), 500),
    ((1, 2, 777, 128), 776),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-w{c[1]}")
def test_window_forward_backward(case, dtype):
    shape, win = case
    B, H, N, d = shape
    seed = 900 + N + win + d
    _announce("window", shape, win, dtype, "seed", seed)
    E = _api()
    inp = synth.qkvdo(seed, shape, dtype)
    q, k, v, do = (upload(inp[x + "_raw"], dtype) for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd_window(q, k, v, win, scale=scale)
    dq, dk, dv = E.attn_bwd_window(q, k, v, o, do, lse, win, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = WO.forward_window(inp["q"], inp["k"], inp["v"], win, scale)
    g_r = WO.backward_window(inp["q"], inp["k"], inp["v"], inp["do"], win, scale)
    assert_close(download(o), o_r, dtype, "O")
    assert_close(download(lse), lse_r, dtype, "LSE")
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
        assert_close(download(got), ref, dtype, name)


def test_window_at_full_size():
    """N = 4096, d = 128, window 1024 (the forward and dQ workgroups start
    inside the window of their first row; dK/dV blocks end at the window of
    their last key), every element against the oracle."""
    shape, win = (1, 2, 4096, 128), 1024
    _announce("window full size", shape, win)
    E = _api()
    inp = synth.qkvdo(4242, shape, "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    o, lse = E.attn_fwd_window(q, k, v, win)
    dq, dk, dv = E.attn_bwd_window(q, k, v, o, do, lse, win)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(128)
    o_r, lse_r = WO.forward_window(inp["q"], inp["k"], inp["v"], win, scale)
    g_r = WO.backward_window(inp["q"], inp["k"], inp["v"], inp["do"], win, scale)
    assert_close(download(o), o_r, "bf16", "O")
    assert_close(download(lse), lse_r, "bf16", "LSE")
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
        assert_close(download(got), ref, "bf16", name)


def test_wide_window_is_the_causal_path():
    shape = (2, 2, 333, 128)
    _announce("window >= N", shape)
    E = _api()
    inp = synth.qkvdo(83, shape, "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    o1, l1 = E.attn_fwd(q, k, v, causal=True)
    g1 = E.attn_bwd(q, k, v, o1, do, l1, causal=True)
    for win in (333, 10 ** 6):
        o2, l2 = E.attn_fwd_window(q, k, v, win)
        g2 = E.attn_bwd_window(q, k, v, o2, do, l2, win)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
