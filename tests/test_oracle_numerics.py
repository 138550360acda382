"""Pins for the oracle's storage-type conversions against torch's casts and
hand-built ties (round to nearest, ties to even)."""
import numpy as np
import torch

from oracle import numerics as nm


def test_bf16_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000),
        rng.standard_normal(1000).astype(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38, -3.3e38], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nm.f32_to_bf16(x), want)


def test_bf16_ties_to_even_and_widening():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20],
                 dtype=np.float32)
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7], dtype=np.float32)
    assert np.array_equal(nm.round_bf16(x), want)
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], dtype=np.uint16)
    assert np.array_equal(nm.bf16_to_f32(bits),
                          torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_f16_matches_torch_including_subnormals():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float16).numpy()
    got = nm.f16(x)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
