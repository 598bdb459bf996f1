"""Pins for the oracle's bf16 conversions and for the input generator's rounding.

The expected bit patterns are fixed by the bf16 format itself (sign, 8 exponent
bits, 7 mantissa bits, round to nearest with ties to even); torch's own bf16
conversion is an independent implementation used as a second witness."""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits
from workloads import bf16_bits_from_f32

CASES = [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (np.inf, 0x7F80), (-np.inf, 0xFF80),
    (2.0 ** -126, 0x0080),               # smallest normal
    (2.0 ** -133, 0x0001),               # smallest subnormal
    (float.fromhex("0x1.fep127"), 0x7F7F),  # largest finite
    (1 + 2.0 ** -8, 0x3F80),             # tie between 1 and 1+2^-7: even mantissa wins
    (1 + 3 * 2.0 ** -8, 0x3F82),         # tie between 0x3F81 and 0x3F82: even wins
    (1 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie: rounds up
    (1 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),  # just below the tie: rounds down
    (3 * 2.0 ** -134, 0x0002),           # subnormal tie 1.5 ulp -> 2 (even)
    (2.0 ** -134, 0x0000),               # half the smallest subnormal ties to +0
    (float.fromhex("0x1.ff0p127"), 0x7F80),  # largest finite + half spacing ties to inf
    (float.fromhex("0x1.fefp127"), 0x7F7F),  # below that tie stays finite
    (0.1, 0x3DCD), (-3.140625, 0xC049),
]


@pytest.mark.parametrize("x,bits", CASES)
def test_known_patterns(x, bits):
    assert int(f64_to_bf16_bits(np.array([x]))[0]) == bits


def test_nan_is_quiet_nan():
    assert int(f64_to_bf16_bits(np.array([np.nan]))[0]) == 0x7FC0


def test_decode_all_patterns_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zeros
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_roundtrip_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    ok = ~np.isnan(v)
    assert np.array_equal(f64_to_bf16_bits(v[ok]), bits[ok])


def test_matches_torch_on_float32_inputs():
    # float32 inputs: torch rounds float32 -> bf16 once, so both must agree exactly
    g = np.random.default_rng(7)
    x = (g.standard_normal(200000) * np.exp2(g.integers(-140, 120, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(x.astype(np.float64)), ref)


def test_single_rounding_from_f64():
    # a value that double rounding through float32 would get wrong: 1 + 2^-8 + 2^-30
    # rounds to float32 1 + 2^-8 (a bf16 tie -> 1.0), but directly it is above the tie.
    x = 1 + 2.0 ** -8 + 2.0 ** -30
    assert int(f64_to_bf16_bits(np.array([x]))[0]) == 0x3F81


def test_generator_rounding_matches_torch():
    g = np.random.default_rng(3)
    x = g.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), ref)
