"""GPU parity of the forward pass against the float64 oracle (through the C ABI)."""

import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.gpu_util import assert_close, download, upload

pytestmark = [pytest.mark.gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


def _run_fwd(inp, dtype, causal, scale):
    E = _api()
    q, k, v = (upload(inp[x + "_raw"], dtype) for x in ("q", "k", "v"))
    o, lse = E.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return download(o), download(lse)


SMALL = [
    # (B, H, N, d): several tiles and ragged tails
    (1, 1, 1, 64),
    (1, 2, 2, 64),
    (2, 1, 3, 128),
    (1, 3, 63, 64),
    (2, 2, 127, 128),
    (1, 2, 129, 64),
    (2, 3, 300, 128),
    (1, 2, 513, 64),
    (1, 1, 777, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL)
def test_forward_small_shapes(shape, causal, dtype):
    seed = 1000 + sum(shape) + 7 * causal
    _announce("fwd", shape, dtype, "causal" if causal else "full", "seed", seed)
    inp = synth.qkvdo(seed, shape, dtype, with_do=False)
    scale = 1.0 / math.sqrt(shape[3])
    o, lse = _run_fwd(inp, dtype, causal, scale)
    o_ref, lse_ref = A.forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_close(o, o_ref, dtype, "O")
    assert_close(lse, lse_ref, dtype, "LSE")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scale", [1.0, 0.05, -0.3])
def test_forward_explicit_scale(scale, dtype):
    shape = (1, 2, 200, 64)
    _announce("fwd scale", scale, dtype)
    inp = synth.qkvdo(77, shape, dtype, with_do=False)
    o, lse = _run_fwd(inp, dtype, True, scale)
    o_ref, lse_ref = A.forward(inp["q"], inp["k"], inp["v"], True, scale)
    assert_close(o, o_ref, dtype, "O")
    assert_close(lse, lse_ref, dtype, "LSE")


def _pad_features(x, d):
    out = np.zeros(x.shape[:-1] + (d,), dtype=np.float32)
    out[..., : x.shape[-1]] = x
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_paper_notes_worked_example_on_gpu(dtype):
    """Q = I, K = [[1,2],[3,4]], V = I with scale 1, features zero-padded to 64."""
    with open(os.path.join(GOLDEN, "paper_notes_worked_example.json")) as f:
        g = json.load(f)
    E = _api()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (
        torch.from_numpy(_pad_features(np.array(g[x], dtype=np.float32), 64))[None, None].to("cuda", tdt)
        for x in ("Q", "K", "V")
    )
    o, lse = E.attn_fwd(q, k, v, causal=False, scale=1.0)
    o = download(o)[0, 0, :, :2]
    lse = download(lse)[0, 0]
    tol = 0.5 * 10 ** (-g["printed_decimals"]) + (4e-3 if dtype == "bf16" else 1e-6)
    np.testing.assert_allclose(o, np.array(g["O"]), atol=tol, rtol=0)
    p0 = 1.0 / (1.0 + math.e**2)
    exact_o = np.array([[p0, 1 - p0], [p0, 1 - p0]])
    exact_lse = np.array([3 + math.log1p(math.exp(-2)), 4 + math.log1p(math.exp(-2))])
    assert_close(o, exact_o, dtype, "O")
    assert_close(lse, exact_lse, dtype, "LSE")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_aicassindra_tiny_example_on_gpu(dtype):
    """One query, scores [1, 3, 2, 5] (d = 1 zero-padded to 64), scale 1."""
    with open(os.path.join(GOLDEN, "aicassindra_tiny_example.json")) as f:
        g = json.load(f)
    E = _api()
    scores = np.concatenate([np.array(b, dtype=np.float32) for b in g["blocks"]])
    n = scores.size
    q = np.zeros((n, 64), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((n, 64), np.float32)
    k[:, 0] = scores
    v = np.zeros((n, 64), np.float32)
    v[:, :n] = np.eye(n)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(x)[None, None].to("cuda", tdt) for x in (q, k, v))
    o, lse = E.attn_fwd(tq, tk, tv, causal=False, scale=1.0)
    lse = download(lse)[0, 0]
    o = download(o)[0, 0]
    # The denominator over all four scores, relative to the max 5, is 1.203.
    tol = 0.5 * 10 ** (-g["printed_decimals"]) + 1e-5
    assert abs(math.exp(lse[0] - 5.0) - g["one_shot_l"]) <= tol
    p = np.exp(scores - (5.0 + math.log(float(np.exp(scores - 5.0).sum()))))
    assert_close(o[0, :n], p, dtype, "P row")
    assert_close(lse, np.full(n, 5.0 + math.log(float(np.exp(scores - 5.0).sum()))), dtype, "LSE")


# ---------------------------------------------------------------------------
# The measured workloads at their full sizes
# ---------------------------------------------------------------------------


def _sampled_rows_check(w, inp, o, lse, count, seed):
    pairs = synth.sample_pairs(seed, w.b * w.h, w.n, count)
    scale = 1.0 / math.sqrt(w.d)
    qf = inp["q"].reshape(w.b * w.h, w.n, w.d)
    kf = inp["k"].reshape(w.b * w.h, w.n, w.d)
    vf = inp["v"].reshape(w.b * w.h, w.n, w.d)
    of = o.reshape(w.b * w.h, w.n, w.d)
    lf = lse.reshape(w.b * w.h, w.n)
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for hd in np.unique(pairs[:, 0]):
        rows = pairs[pairs[:, 0] == hd, 1]
        ro, rl = A.forward_rows(qf[hd], kf[hd], vf[hd], rows, w.causal, scale)
        got_o.append(of[hd, rows])
        ref_o.append(ro)
        got_l.append(lf[hd, rows])
        ref_l.append(rl)
    assert_close(np.concatenate(got_o), np.concatenate(ref_o), w.dtype, f"{w.name} O (sampled rows)")
    assert_close(np.concatenate(got_l), np.concatenate(ref_l), w.dtype, f"{w.name} LSE (sampled rows)")


@pytest.mark.parametrize(
    "name",
    ["fp32_n256_d64", "gpt2s_n1024_d64_causal", "n4096_d128", "n4096_d128_causal", "bwd_n2048_d64_causal",
     "long_n65536_d64_causal"],
)
def test_forward_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    _announce("fwd full size", w)
    inp = synth.qkvdo(w.seed, w.shape, w.dtype, with_do=False)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = _run_fwd(inp, w.dtype, w.causal, scale)
    if w.b * w.h * w.n <= 1024 * 96:
        o_ref, lse_ref = A.forward(inp["q"], inp["k"], inp["v"], w.causal, scale)
        assert_close(o, o_ref, w.dtype, f"{name} O")
        assert_close(lse, lse_ref, w.dtype, f"{name} LSE")
    else:
        _sampled_rows_check(w, inp, o, lse, 512, w.seed + 1)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
