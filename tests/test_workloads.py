"""The seeded input module: bf16 storage conversion and determinism."""

import numpy as np
import pytest
import torch

from matrix_optimizer_step_muon_amd import workloads as wl


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e-3,
                        np.array([1.0, -2.5, 1e-40, 3.4e38, 0.0, -0.0], np.float32),
                        np.array([0x3F808000, 0x3F818000, 0x3F80FFFF], np.uint32).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(wl.f32_to_bf16_bits(x), want)
    back = wl.bf16_bits_to_f32(want)
    np.testing.assert_array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_ties_to_even():
    bits = np.array([0x3F808000, 0x3F818000], np.uint32).view(np.float32)
    np.testing.assert_array_equal(wl.f32_to_bf16_bits(bits), np.array([0x3F80, 0x3F82], np.uint16))


def test_nan_stays_nan():
    assert np.isnan(wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_generation_is_seeded_and_per_matrix():
    w = wl.WORKLOADS["qwen3_1p7b_layer"]
    a = wl.generate_matrix(w, 1)
    b = wl.generate(w, [1])[0]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert a[0].dtype == np.uint16 and a[0].shape == (1024, 2048)
    g = wl.stored_to_f64(a[1], "bf16")
    assert 0.9e-3 < g.std() < 1.1e-3


def test_workload_sizes():
    assert wl.WORKLOADS["qwen3_32b_layer"].numel == 487_587_840
    assert len(wl.WORKLOADS["qwen3_1p7b_28_layers"].shapes) == 196
    assert len(wl.WORKLOADS["qwen3_32b_rank_share"].shapes) == 17
