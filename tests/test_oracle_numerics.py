"""Pins for oracle.numerics against torch's CPU library routines."""

import numpy as np
import torch

from oracle import numerics


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45],
                 dtype=np.float32),
    ])
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (np.arange(0x3F800000, 0x3F800000 + (64 << 16), 1 << 16,
                      dtype=np.uint32) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = numerics.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_nan_stays_nan():
    assert np.isnan(numerics.bf16_round(np.array([np.nan], np.float32)))[0]


def test_gelu_matches_torch_fp64():
    x = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(numerics.gelu(x), ref, rtol=1e-14, atol=1e-15)


def test_gelu_closed_forms():
    x = np.linspace(-5, 5, 101)
    assert numerics.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(numerics.gelu(x) - numerics.gelu(-x), x, atol=1e-14)
