"""The online-softmax rescale on the GPU, forced by the inputs.

The forward kernel computes each 32-key unit's probabilities against the
current reference max and takes the unit's max, raises the reference and
rescales the output and the running sum (``settle`` in
csrc/attn_fwd_bf16.hip) only when some lane's unit sum exceeds 2^8.  On
standard-normal inputs at scale 1/sqrt(d) that happens essentially only on a
row's first unit, so these tests build inputs whose running max climbs by more
than 8 / (scale log2 e) inside rows -- the running-max / running-sum update
of the aicassindra page ("Online softmax: the running-max, running-sum idea";
"A tiny worked example") and of "Tiling: Block-by-Block Softmax" (Paper
Notes):

* a key ramp (feature 0 of key j grows with j): every whole unit after the
  first raises every row's max past the gate (forward, both masks);
* peaked rows (scores rise like a cosine toward a key chosen per query; every
  eighth query peaks in the last tile, and under the causal mask a row whose
  peak lies beyond it has its max at its last key): about one unit in seven
  takes the branch, in about three rows of four (forward and backward, both
  masks; the backward recomputes P from the LSE these rows produce).  The
  two score-shaping features carry large values common to the keys (and
  queries) a row attends to, which multiply the bf16 rounding of dS, of O
  (from which D is formed) and of the outputs into the gradients; the query
  side carries 3x the key side's magnitude and dO is scaled by 1/512, so that
  a CPU model of exactly that rounding stays inside the tolerance (relative
  Frobenius about 0.005, max abs below 0.005).  With equal magnitudes and
  dO ~ N(0, 1/16) the same model gives dQ 0.047 max abs, as the GPU did.

tests/test_synth.py checks on the CPU that the inputs do cross the gate.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.gpu_util import assert_close, download, oracle_map, upload

pytestmark = [pytest.mark.gpu]

N = 4096


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_key_ramp_rescales_every_unit(d, causal):
    shape = (1, 2, N, d)
    _announce("fwd key ramp", shape, "causal" if causal else "full")
    E = _api()
    inp = synth.ramp_inputs(31 + d, shape)
    scale = 1.0 / math.sqrt(d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = download(o), download(lse)
    refs = oracle_map(lambda hd: A.forward_head(inp["q"][0, hd], inp["k"][0, hd], inp["v"][0, hd], causal, scale),
                      range(2))
    assert_close(o[0], np.stack([r[0] for r in refs]), "bf16", "O")
    assert_close(lse[0], np.stack([r[1] for r in refs]), "bf16", "LSE")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_backward_peaked_rows(d, causal):
    shape = (1, 2, N, d)
    _announce("fwd+bwd peaked rows", shape, "causal" if causal else "full")
    E = _api()
    scale = 1.0 / math.sqrt(d)
    inp = synth.peaked_inputs(41 + d, shape, 220.0 / scale, do_scale=1.0 / 512)
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    o, lse = E.attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = E.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = [download(x)[0] for x in (o, lse, dq, dk, dv)]

    def head(hd):
        a = [inp[x][0, hd] for x in ("q", "k", "v", "do")]
        return list(A.forward_head(*a[:3], causal, scale)) + list(A.backward_head(*a, causal, scale))

    refs = oracle_map(head, range(2))
    for i, name in enumerate(("O", "LSE", "dQ", "dK", "dV")):
        assert_close(got[i], np.stack([r[i] for r in refs]), "bf16", name)
