"""Host checks of the seeded input generator (no attention arithmetic here)."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate(
        [
            rng.standard_normal(100000).astype(np.float32),
            np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], dtype=np.float32),
        ]
    )
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_reproducible_and_exact():
    a = synth.qkvdo(7, (1, 2, 5, 4), "bf16")
    b = synth.qkvdo(7, (1, 2, 5, 4), "bf16")
    for name in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[name + "_raw"], b[name + "_raw"])
        np.testing.assert_array_equal(a[name], synth.bf16_bits_to_f32(a[name + "_raw"]).astype(np.float64))
    f = synth.qkvdo(7, (1, 2, 5, 4), "fp32")
    # Same underlying draws, before rounding.
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(f["q_raw"]), a["q_raw"])


def test_sample_pairs_are_distinct_and_in_range():
    p = synth.sample_pairs(6, 8, 65536, 512)
    assert p.shape == (512, 2)
    assert len({(int(h), int(r)) for h, r in p}) == 512
    assert p[:, 0].min() >= 0 and p[:, 0].max() < 8
    assert p[:, 1].min() >= 0 and p[:, 1].max() < 65536


def _gate_crossings(q, k, scale, causal):
    """Per (row, 32-key unit): does the unit's max exceed the running max of
    the earlier units by more than 8 / (scale log2 e), so that one
    probability taken against the old max exceeds 2^8?"""
    import math

    n = q.shape[0]
    s = q @ k.T
    if causal:
        s[np.triu_indices(n, 1)] = -np.inf
    um = s.reshape(n, n // 32, 32).max(-1)
    prev = np.concatenate([np.full((n, 1), -np.inf), np.maximum.accumulate(um, axis=1)[:, :-1]], axis=1)
    ok = np.isfinite(um) & np.isfinite(prev)
    return ((um - prev) * scale * math.log2(math.e) > 8) & ok, ok


def test_rescale_inputs_cross_the_gate():
    """The inputs of tests/test_rescale_gpu.py force the forward's rescale
    inside rows: the key ramp in every whole unit after a row's first, the peaked
    rows in at least a tenth of the units and in most rows."""
    import math

    n = 4096
    for d in (64, 128):
        scale = 1.0 / math.sqrt(d)
        r = synth.ramp_inputs(31 + d, (1, 1, n, d))
        p = synth.peaked_inputs(41 + d, (1, 1, n, d), 220.0 / scale, do_scale=1.0 / 512)
        for causal in (False, True):
            cross, ok = _gate_crossings(r["q"][0, 0], r["k"][0, 0], scale, causal)
            # (Under the causal mask a row's diagonal unit may hold only a few
            # keys past the previous unit's max; every whole unit crosses.)
            whole = 32 * np.arange(n // 32)[None, :] + 31 <= np.arange(n)[:, None] if causal else ok
            assert cross[ok & whole].all() and (ok & whole).sum() >= ok.sum() - n
            cross, ok = _gate_crossings(p["q"][0, 0], p["k"][0, 0], scale, causal)
            assert cross.sum() >= 0.1 * ok.sum() and cross.any(1).sum() >= n // 2
