"""Pin of the oracle's bf16 rounding against torch's CPU cast (round to nearest even)."""
import numpy as np
import torch

from oracle.numerics import round_bf16, bf16_bits, bf16_to_f64


def _torch_bf16(x64):
    # torch casts binary32 -> bf16 with RNE; feed values that are exact in binary32
    return torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_matches_torch_on_random_binary32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1.0, 30.0, 1e5)])
    x = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(round_bf16(x), _torch_bf16(x))


def test_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even); 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 2.0**-130 * 1.5])
    assert np.array_equal(round_bf16(x), _torch_bf16(x))
    assert round_bf16(np.array([1 + 2.0**-8]))[0] == 1.0


def test_overflow_subnormal_and_specials():
    x = np.array([3.4e38, 3.39e38, 1e-40, -1e-42, 0.0, -0.0, np.inf, -np.inf])
    assert np.array_equal(round_bf16(x), _torch_bf16(x))
    assert np.isnan(round_bf16(np.array([np.nan]))[0])


def test_bits_roundtrip():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000)
    assert np.array_equal(bf16_to_f64(bf16_bits(x)), round_bf16(x))
