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
