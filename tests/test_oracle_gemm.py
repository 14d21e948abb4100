"""Pins for the oracle GEMM and glue: exact rational arithmetic on tiny shapes, closed
forms, and the BF16 rounding rule checked on values whose rounding is known."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm
from lossless_bf16_weight_amd import synth


def frac_bf16(bits):
    b = int(bits)
    s, e, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
    assert e != 255
    v = Fraction(m, 128) * Fraction(2) ** (-126) if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if s else v


@pytest.mark.parametrize("m,n,k,seed", [(1, 3, 64, 0), (3, 5, 128, 1), (2, 4, 64, 2)])
def test_gemm_ref_equals_exact_rational(m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = synth.gaussian_bf16(rng, (m, k), 1.0)
    w = synth.gaussian_bf16(rng, (n, k), 0.02)
    y, s = gemm.gemm_ref(x, w)
    for i in range(m):
        for j in range(n):
            exact = sum(frac_bf16(x[i, c]) * frac_bf16(w[j, c]) for c in range(k))
            absum = sum(abs(frac_bf16(x[i, c]) * frac_bf16(w[j, c])) for c in range(k))
            assert abs(Fraction(y[i, j]) - exact) <= Fraction(k, 2 ** 52) * absum
            assert abs(Fraction(s[i, j]) - absum) <= Fraction(k, 2 ** 52) * absum


def test_gemm_ref_multi_equals_exact_rational():
    """The several-inputs form, pinned the same way: exact rational dot products."""
    rng = np.random.default_rng(9)
    w = synth.gaussian_bf16(rng, (3, 64), 0.02)
    xs = [synth.gaussian_bf16(rng, (m, 64), 1.0) for m in (1, 2)]
    for x, (y, s) in zip(xs, gemm.gemm_ref_multi(xs, w)):
        for i in range(x.shape[0]):
            for j in range(3):
                exact = sum(frac_bf16(x[i, c]) * frac_bf16(w[j, c]) for c in range(64))
                absum = sum(abs(frac_bf16(x[i, c]) * frac_bf16(w[j, c])) for c in range(64))
                assert abs(Fraction(y[i, j]) - exact) <= Fraction(64, 2 ** 52) * absum
                assert abs(Fraction(s[i, j]) - absum) <= Fraction(64, 2 ** 52) * absum


def test_gemm_orientation_and_identity():
    """W rows that hold a single 1.0 select the matching input: y[:, j] = x[:, j]."""
    rng = np.random.default_rng(3)
    x = synth.gaussian_bf16(rng, (4, 64), 1.0)
    w = np.zeros((64, 64), np.uint16)
    w[np.arange(64), np.arange(64)] = 0x3F80            # 1.0
    y, s = gemm.gemm_ref(x, w)
    assert np.array_equal(y, gemm.bf16_to_f64(x))
    assert np.array_equal(s, np.abs(gemm.bf16_to_f64(x)))


def test_bf16_decoding_of_known_values():
    assert gemm.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x0001]))[:5].tolist() == \
        [1.0, -2.0, 0.0, -0.0, 0.25]
    assert gemm.bf16_to_f64(np.array([0x0001]))[0] == 2.0 ** -133


def test_within_bound_definition():
    y_ref = np.array([1.0, 0.0, 2.0])
    s = np.array([10.0, 0.0, 1.0])
    assert gemm.within_bound(np.array([1.0099, 0.0, 2.0]), y_ref, s).tolist() == [True, True, True]
    assert gemm.within_bound(np.array([1.0101, 1e-30, 2.002]), y_ref, s).tolist() == [False, False, False]


def test_rne_rounding_known_cases():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {one: 0x3F80, one + ulp / 2: 0x3F80,           # tie -> even (mantissa 0)
             one + 3 * ulp / 2: 0x3F82,                      # tie -> even (mantissa 2)
             one + ulp / 2 + 2 ** -20: 0x3F81, -2.0: 0xC000, 0.0: 0x0000}
    for v, bits in cases.items():
        assert int(gemm.f64_to_bf16_rne(np.array([v]))[0]) == bits, v


def test_swiglu_and_rmsnorm_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 20.0])
    u = np.array([3.0, 2.0, 2.0, 1.0])
    h = gemm.bf16_to_f64(gemm.swiglu_ref(g, u))
    silu = g / (1 + np.exp(-g))
    assert h[0] == 0.0
    assert np.allclose(h, silu * u, rtol=2 ** -8)
    y = np.array([[3.0, 4.0, 0.0, 0.0]])                   # mean square 25/4
    x = gemm.bf16_to_f64(gemm.rmsnorm_ref(y, eps=0.0))
    assert np.allclose(x, [[1.2, 1.6, 0.0, 0.0]], rtol=2 ** -8)
