"""Pins for the oracle's numerics: exact bf16 values, the fp64 matmul against
exact rational sums, bf16 rounding on every bf16 value and every midpoint, and
SiLU identities."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import numerics
import workloads


def test_bf16_values_exact():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x8001, 0x0080, 0x7F7F, 0x7F80, 0xFF80,
                     0x3F81, 0x0000, 0x8000], np.uint16)
    expect = [1.0, -2.0, 2.0 ** -133, -(2.0 ** -133), 2.0 ** -126,
              (2 - 2 ** -7) * 2.0 ** 127, np.inf, -np.inf, 1 + 2 ** -7, 0.0, -0.0]
    got = numerics.bf16_to_f64(bits)
    for g, e in zip(got, expect):
        assert g == e
    assert np.signbit(got[-1])


def _frac_of_bf16(b):
    b = int(b)
    s = -1 if b & 0x8000 else 1
    E = (b >> 7) & 0xFF
    m = b & 0x7F
    if E == 0:
        return s * Fraction(m, 2 ** 133)
    return s * Fraction(128 + m, 2 ** 7) * Fraction(2) ** (E - 127)


def test_matmul_equals_exact_rational_sums():
    rng = np.random.default_rng(11)
    W = workloads.gaussian_weights(rng, 5, 64, 0.02, 0.05, 1.0)
    X = workloads.gaussian_activations(rng, 3, 64)
    Y = numerics.matmul(W, X)
    S = numerics.abs_bound(W, X)
    for b in range(3):
        for r in range(5):
            exact = sum(_frac_of_bf16(W[r, c]) * _frac_of_bf16(X[b, c]) for c in range(64))
            bound = sum(abs(_frac_of_bf16(W[r, c]) * _frac_of_bf16(X[b, c])) for c in range(64))
            assert abs(Fraction(Y[b, r]) - exact) <= Fraction(64, 2 ** 52) * bound
            assert abs(Fraction(S[b, r]) - bound) <= Fraction(64, 2 ** 52) * bound
    Yr, Sr = numerics.matmul_rows(W, X, [4, 1])
    assert np.array_equal(Yr[:, 0], Y[:, 4]) and np.array_equal(Sr[:, 1], S[:, 1])


def test_f64_to_bf16_identity_on_every_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = numerics.bf16_to_f64(bits)
    back = numerics.f64_to_bf16_bits(vals)
    finite = np.isfinite(vals)
    assert np.array_equal(back[finite], bits[finite])
    inf = np.isinf(vals)
    assert np.array_equal(back[inf], bits[inf])
    nan = np.isnan(vals)
    assert np.all(np.isnan(numerics.bf16_to_f64(back[nan])))


def test_f64_to_bf16_midpoints_round_to_even():
    # midpoint between consecutive positive finite bf16 values a < b
    bits = np.arange(0x0000, 0x7F7F, dtype=np.uint16)
    a = numerics.bf16_to_f64(bits)
    b = numerics.bf16_to_f64(bits + 1)
    mid = (a + b) / 2       # exact in fp64
    got = numerics.f64_to_bf16_bits(mid)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    got_neg = numerics.f64_to_bf16_bits(-mid)
    assert np.array_equal(got_neg, even | 0x8000)
    # just above / below the midpoint
    assert np.array_equal(numerics.f64_to_bf16_bits(np.nextafter(mid, np.inf)), bits + 1)
    assert np.array_equal(numerics.f64_to_bf16_bits(np.nextafter(mid, 0)), bits)


def test_f64_to_bf16_agrees_with_fp32_rne_rounding():
    # the input generator rounds fp32 -> bf16 with an integer-add trick;
    # the oracle rounds the exact value; they must agree on every finite fp32
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    x = np.concatenate([x, x * 1e-38, x * 1e30]).astype(np.float32)
    assert np.array_equal(numerics.f64_to_bf16_bits(x.astype(np.float64)),
                          workloads.f32_to_bf16_bits(x))


def test_f64_to_bf16_overflow():
    # largest finite bf16 is 255 * 2^120 (odd mantissa); the midpoint to
    # 2^128 is one half-ulp (2^119) above it and ties to even -> infinity
    big = numerics.bf16_to_f64(np.array([0x7F7F], np.uint16))[0]
    assert big == 255 * 2.0 ** 120
    mid = big + 2.0 ** 119
    assert numerics.f64_to_bf16_bits(np.array([mid]))[0] == 0x7F80
    assert numerics.f64_to_bf16_bits(np.array([np.nextafter(mid, 0)]))[0] == 0x7F7F
    assert numerics.f64_to_bf16_bits(np.array([-mid]))[0] == 0xFF80


def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    s = numerics.silu(z)
    assert numerics.silu(np.array([0.0]))[0] == 0.0
    # silu(z) - silu(-z) = z
    assert np.allclose(s - numerics.silu(-z), z, rtol=0, atol=1e-12)
    # silu(z) = z * sigmoid(z); sigmoid(z) = e^z / (1 + e^z), well conditioned for z < 0
    neg = z < 0
    assert np.allclose(s[neg], z[neg] * np.exp(z[neg]) / (1 + np.exp(z[neg])), rtol=1e-13, atol=0)
    assert np.allclose(s, z * 0.5 * (1 + np.tanh(z / 2)), rtol=0, atol=1e-13)
    h = numerics.silu_mul(np.array([1.0, -2.0]), np.array([3.0, 0.5]))
    assert h[0] == pytest.approx(3.0 / (1 + np.exp(-1.0)))
    assert h[1] == pytest.approx(0.5 * -2.0 / (1 + np.exp(2.0)))
