"""Pins of the oracle's number formats and bit packing (hand-computed values)."""
import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("x,expect", [
    (1 + 2 ** -11, 1.0),                           # exact tie -> even
    (1 + 2 ** -11 + 2 ** -40, 1 + 2 ** -10),       # just above the tie (one rounding, not via fp32)
    (1 + 3 * 2 ** -11, 1 + 2 ** -9),               # tie -> even (odd 1+2^-10 loses)
    (65519.99, 65504.0),                           # largest finite
    (2.0 ** -24, 2.0 ** -24),                      # smallest subnormal
    (2.0 ** -25, 0.0),                             # half of it: tie -> even (0)
    (3 * 2.0 ** -26, 2.0 ** -24),                  # above the half
    (-0.7, -0.7001953125),
])
def test_fp16_rne(x, expect):
    assert float(O.fp16_rne(np.float64(x))) == expect


def test_fp16_overflow():
    assert np.isinf(O.fp16_rne(np.float64(65520.0)))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (1 + 2 ** -8, 0x3F80),          # tie -> even
    (1 + 3 * 2 ** -8, 0x3F82), (1 + 2 ** -8 + 2 ** -30, 0x3F81),  # tie -> even / above tie
    (0.0, 0x0000), (3.0, 0x4040),
])
def test_bf16_rne(x, bits):
    assert int(O.f64_to_bf16(np.float64(x))) == bits


def test_bf16_roundtrip_all_finite_patterns():
    b = np.arange(65536, dtype=np.uint16)
    v = O.bf16_to_f64(b)
    fin = np.isfinite(v) & (v != 0)
    assert np.array_equal(O.f64_to_bf16(v[fin]), b[fin])


def test_pack_k_codes_examples():
    c = np.zeros(128, np.uint8)
    c[:4] = [1, 2, 3, 0]
    c[4:8] = [3, 3, 3, 3]
    c[127] = 2
    b = O.pack_k_codes(c)
    assert b[0] == 0x39 and b[1] == 0xFF and b[31] == 0x80 and b[2:31].sum() == 0
    rng = np.random.default_rng(0)
    r = rng.integers(0, 4, (5, 128)).astype(np.uint8)
    assert np.array_equal(O.unpack_k_codes(O.pack_k_codes(r)), r)
