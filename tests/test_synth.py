"""Input generators: bf16 rounding matches torch's round-to-nearest-even, seeds are stable."""

import numpy as np
import torch

from exact_blockwise_long_amd import synth


def test_bf16_rounding_matches_torch():
    g = synth.rng(7)
    x = (g.standard_normal(100000, dtype=np.float32) * np.float32(3.0)).astype(np.float32)
    # include exact ties and extremes
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1e-40, 3.0e38], dtype=np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_inputs_are_reproducible():
    a = synth.normal(synth.rng(3), (4, 5), 0.5, "bf16")
    b = synth.normal(synth.rng(3), (4, 5), 0.5, "bf16")
    assert a.sha256() == b.sha256()
    assert a.f64().dtype == np.float64
