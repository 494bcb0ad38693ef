"""The seeded input recipe: bf16 rounding, determinism and distributions."""
import numpy as np
import torch

from seeded_inputs import WORKLOADS, round_to_bf16_bits, bf16_bits_to_float32, slice_f32, slice_values


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.0078125, 0.0, -0.0, 65504.0], np.float32)])
    ours = round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_float32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_are_deterministic_and_distinct():
    w = WORKLOADS[2].with_(n_frames=2, tokens_per_frame=64)
    a = slice_f32(w, "q", 0, 3)
    assert np.array_equal(a, slice_f32(w, "q", 0, 3))
    assert not np.array_equal(a, slice_f32(w, "q", 0, 4))
    assert not np.array_equal(a, slice_f32(w, "k", 0, 3))


def test_distributions():
    w = WORKLOADS[3].with_(n_frames=4, tokens_per_frame=256)
    q = slice_f32(w, "q", 0, 0)
    rms = np.sqrt(np.mean(q.astype(np.float64) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=1e-5)
    tv = slice_f32(w, "tv", 0, 0)
    assert abs(tv.std() - 0.1) < 0.002
    v = slice_f32(w, "v", 0, 0)
    assert abs(v.std() - 1.0) < 0.01
    vals = slice_values(w, "v", 0, 0)
    assert np.array_equal(vals, bf16_bits_to_float32(round_to_bf16_bits(v)).astype(np.float64))
    t5 = slice_f32(WORKLOADS[5].with_(n_frames=4, tokens_per_frame=256), "tk", 0, 0)
    assert abs(t5.std() - 0.05) < 0.001
