"""CPU model of the backward kernels' rounding, justifying the hi + lo split.

The bf16 backward rounds the probabilities P (and dS) to bf16 before they
enter the dV (and dK) matrix products.  This test models exactly that
arithmetic in float64 around the oracle's exact values: with a single bf16
rounding of P, the largest dV error of a ragged causal case exceeds the 2e-2
tolerance (the GPU measured the same 0.0203); with P = hi + lo (two bf16
values) the error falls to the output-rounding floor.
"""

import math

import numpy as np
import torch

import synth
from oracle import attention as A


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _hilo(x):
    hi = _bf16(x)
    return hi + _bf16(x - hi)


def test_single_bf16_probabilities_exceed_tolerance_and_hilo_does_not():
    shape, causal = (2, 2, 129, 128), True
    seed = 2000 + sum(shape) + 11
    inp = synth.qkvdo(seed, shape, "bf16")
    scale = 1.0 / math.sqrt(shape[3])
    q, k, do = inp["q"], inp["k"], inp["do"]
    _, lse = A.forward(q, k, inp["v"], causal, scale)
    _, _, dv_ref = A.backward(q, k, inp["v"], do, causal, scale)
    err_bf16, err_hilo, err_floor = 0.0, 0.0, 0.0
    for b in range(shape[0]):
        for h in range(shape[1]):
            p = np.exp(A.scores(q[b, h], k[b, h], scale, causal) - lse[b, h][:, None])
            ref = dv_ref[b, h]
            err_bf16 = max(err_bf16, np.abs(_bf16(_bf16(p).T @ do[b, h]) - ref).max())
            err_hilo = max(err_hilo, np.abs(_bf16(_hilo(p).T @ do[b, h]) - ref).max())
            err_floor = max(err_floor, np.abs(_bf16(ref) - ref).max())
    assert err_bf16 > 2e-2
    assert err_hilo < 1.2 * err_floor + 1e-3
    assert err_hilo < 1.5e-2


def _selective(p, tau=1.0 / 16, tq=32, tk=32, weight=1.0):
    """hi + lo only on 32 x 32 tiles holding a value with weight * |value| >=
    tau, as the kernel does."""
    out = _bf16(p)
    full = _hilo(p)
    for i in range(0, p.shape[0], tq):
        for j in range(0, p.shape[1], tk):
            if weight * np.abs(p[i : i + tq, j : j + tk]).max() >= tau:
                out[i : i + tq, j : j + tk] = full[i : i + tq, j : j + tk]
    return out


def test_selective_split_keeps_the_full_split_accuracy():
    """Splitting only tiles with a probability >= 1/16 loses nothing measurable."""
    shape, causal = (2, 2, 129, 128), True
    seed = 2000 + sum(shape) + 11
    inp = synth.qkvdo(seed, shape, "bf16")
    scale = 1.0 / math.sqrt(shape[3])
    q, k, do = inp["q"], inp["k"], inp["do"]
    _, lse = A.forward(q, k, inp["v"], causal, scale)
    _, _, dv_ref = A.backward(q, k, inp["v"], do, causal, scale)
    err_sel, err_hilo = 0.0, 0.0
    for b in range(shape[0]):
        for h in range(shape[1]):
            p = np.exp(A.scores(q[b, h], k[b, h], scale, causal) - lse[b, h][:, None])
            ref = dv_ref[b, h]
            err_sel = max(err_sel, np.abs(_bf16(_selective(p).T @ do[b, h]) - ref).max())
            err_hilo = max(err_hilo, np.abs(_bf16(_hilo(p).T @ do[b, h]) - ref).max())
    assert err_sel <= err_hilo + 1e-4


def test_selective_split_of_scaled_ds_keeps_the_full_split_accuracy():
    """dS enters dK unscaled and the scale multiplies the sum, so the kernel
    compares scale * |dS| with 1/16: a term's rounding error in dK is then
    bounded as a term's in dV.  That selects few tiles at long N and keeps the
    worst dK error at that of splitting every tile."""
    for shape, causal in (((2, 2, 129, 128), True), ((1, 2, 1000, 128), False)):
        seed = 2000 + sum(shape) + 11
        inp = synth.qkvdo(seed, shape, "bf16")
        scale = 1.0 / math.sqrt(shape[3])
        q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
        o, lse = A.forward(q, k, v, causal, scale)
        _, dk_ref, _ = A.backward(q, k, v, do, causal, scale)
        err_sel, err_hilo = 0.0, 0.0
        for b in range(shape[0]):
            for h in range(shape[1]):
                p = np.exp(A.scores(q[b, h], k[b, h], scale, causal) - lse[b, h][:, None])
                dsum = (do[b, h] * o[b, h]).sum(-1, keepdims=True)
                ds = p * (do[b, h] @ v[b, h].T - dsum)
                ref = dk_ref[b, h]
                sel = _selective(ds, weight=scale)
                err_sel = max(err_sel, np.abs(_bf16(scale * (sel.T @ q[b, h])) - ref).max())
                err_hilo = max(err_hilo, np.abs(_bf16(scale * (_hilo(ds).T @ q[b, h])) - ref).max())
        assert err_sel <= err_hilo + 2e-4, (shape, err_sel, err_hilo)
        assert err_sel < 1e-2


def _peaked_backward_errors(d, causal, q_over_k, do_scale, n=2048):
    """Max abs and relative Frobenius errors of dQ and dK under the kernels'
    rounding (single bf16 dS into dQ; selective hi + lo dS into dK; D from the
    bf16 output O; bf16 outputs) on the peaked inputs of the rescale tests."""
    scale = 1.0 / math.sqrt(d)
    inp = synth.peaked_inputs(41 + d, (1, 1, n, d), 220.0 / scale, q_over_k, do_scale)
    q, k, v, do = (inp[x][0, 0] for x in ("q", "k", "v", "do"))
    o, lse = A.forward_head(q, k, v, causal, scale)
    dq, dk, _ = A.backward_head(q, k, v, do, causal, scale)
    p = np.exp(A.scores(q, k, scale, causal) - lse[:, None])
    ds = p * (do @ v.T - np.sum(do * _bf16(o), 1)[:, None])
    got_q = _bf16(scale * (_bf16(ds) @ k))
    got_k = _bf16(scale * (_selective(ds, weight=scale).T @ q))
    out = []
    for g, r in ((got_q, dq), (got_k, dk)):
        out.append((np.abs(g - r).max(), np.linalg.norm(g - r) / np.linalg.norm(r)))
    return out


def test_peaked_rescale_inputs_stay_inside_the_tolerance():
    """The rescale tests' inputs carry large components common to the keys a
    row attends to.  With equal query and key magnitudes and dO ~ N(0, 1/16)
    the rounding model puts dQ's error past the bf16 tolerance (as the GPU
    measured); with the query side 3x the key side and dO scaled by 1/512 it
    stays well inside."""
    (eq, rq), _ = _peaked_backward_errors(128, True, 1.0, 0.25)
    assert eq > 2e-2 or rq > 1e-2
    for d in (64, 128):
        (eq, rq), (ek, rk) = _peaked_backward_errors(d, True, 9.0, 1.0 / 512)
        assert eq < 0.01 and rq < 0.007 and ek < 0.01 and rk < 0.005
