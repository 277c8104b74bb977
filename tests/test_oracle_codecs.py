"""Pins of the oracle's bf16 codec against the format definition and torch's own cast."""
import numpy as np
import pytest
import torch

from oracle.codecs import bf16_bits_to_f64, f64_to_bf16_bits


def test_decode_known_patterns():
    bits = np.array([0x3F80, 0x40E0, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F], np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == 7.0 and v[2] == -2.0
    assert v[3] == 0.0 and np.signbit(v[4])
    assert v[5] == np.inf and v[6] == -np.inf
    assert v[7] == 2.0 ** -133                       # smallest subnormal
    assert v[8] == (2 - 2 ** -7) * 2.0 ** 127        # largest finite


def test_round_trip_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(f64_to_bf16_bits(v[fin]), bits[fin])


def test_encode_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 cast is an independent nearest-even implementation.
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # include exact ties (low 16 bits = 0x8000) and subnormals
    u[:50_000] = (u[:50_000] & 0xFFFF0000) | 0x8000
    u[50_000:60_000] &= 0x807FFFFF
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_ties_to_even_and_no_double_rounding():
    one = 1.0
    assert bf16_bits_to_f64(f64_to_bf16_bits(one + 2 ** -8)) == 1.0                # tie -> even (down)
    assert bf16_bits_to_f64(f64_to_bf16_bits(one + 3 * 2 ** -8)) == 1 + 2 ** -6     # tie -> even (up)
    # just above a tie: float32 would first round to the tie and then to even (1.0); the
    # direct rounding from float64 must go up.
    assert bf16_bits_to_f64(f64_to_bf16_bits(one + 2 ** -8 + 2 ** -40)) == 1 + 2 ** -7


@pytest.mark.parametrize("x,expect", [(3.4e38, np.inf), (-3.4e38, -np.inf), (3.0e38, (1 + 98 / 128) * 2.0 ** 127), (2.0 ** -134, 0.0),
                                      (1.5 * 2.0 ** -133, 2.0 ** -132)])
def test_overflow_and_subnormal_rounding(x, expect):
    assert bf16_bits_to_f64(f64_to_bf16_bits(x)) == expect
