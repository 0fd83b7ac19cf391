"""Pins for the GEMV oracle: exact rational sums, one-hot and identity cases."""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle.gemv import bf16_bits_to_f64, gemv_rows
from synth import f32_to_bf16_bits, gemv_case


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a bf16 pattern, decoded through the IEEE single layout by hand."""
    (v,) = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))
    return Fraction(v)


@pytest.mark.parametrize("N,K,R,seed", [(8, 32, 1, 1), (16, 24, 4, 2), (5, 40, 3, 3)])
def test_fraction_exact(N, K, R, seed):
    w, x = gemv_case(seed, N, K, R)
    y, s = gemv_rows(w, x)
    for r in range(R):
        for n in range(N):
            exact = sum(bf16_fraction(w[n, k]) * Fraction(float(x[r, k])) for k in range(K))
            mag = sum(abs(bf16_fraction(w[n, k]) * Fraction(float(x[r, k]))) for k in range(K))
            assert abs(Fraction(y[r, n]) - exact) <= mag * Fraction(1, 2**48)
            assert abs(Fraction(s[r, n]) - mag) <= mag * Fraction(1, 2**48)


def test_one_hot_column():
    w, _ = gemv_case(7, 12, 64, 1)
    x = np.zeros((3, 64), dtype=np.float32)
    cols = [0, 17, 63]
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    y, _ = gemv_rows(w, x)
    for r, c in enumerate(cols):
        expect = np.array([float(bf16_fraction(w[n, c])) for n in range(12)])
        assert np.array_equal(y[r], expect)


def test_identity_weights_return_x():
    K = 48
    w = np.zeros((K, K), dtype=np.uint16)
    w[np.arange(K), np.arange(K)] = 0x3F80  # bf16 1.0
    x = np.random.default_rng(0).standard_normal((4, K)).astype(np.float32)
    y, s = gemv_rows(w, x)
    assert np.array_equal(y, x.astype(np.float64))
    assert np.array_equal(s, np.abs(x).astype(np.float64))


def test_row_selection_and_blocking_match_full():
    w, x = gemv_case(11, 300, 64, 2)
    y, s = gemv_rows(w, x)
    sel = np.array([0, 5, 299, 150])
    y2, s2 = gemv_rows(w, x, rows=sel, block=3)
    assert np.array_equal(y2, y[:, sel]) and np.array_equal(s2, s[:, sel])


def test_bf16_decode_and_encode():
    # 1.0, -2.0, smallest normal, +inf patterns decode exactly
    bits = np.array([0x3F80, 0xC000, 0x0080, 0x7F80], dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0**-126 and np.isinf(v[3])
    # round to nearest even on the generator side: 1 + 2^-8 is a tie -> 1.0,
    # 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even), 1 + 2^-8 + 2^-20 rounds up
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20], dtype=np.float32)
    assert list(f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0x3F81]



def test_non_finite_activations_hand_worked():
    """IEEE term-by-term reading of y = sum_k w x for rows holding +-inf or
    NaN, against values worked by hand: an infinite term decides the sign,
    opposite infinities or an infinity times a zero weight give NaN, a NaN
    activation gives NaN everywhere; finite rows are unchanged."""
    inf, nan = np.inf, np.nan
    w = f32_to_bf16_bits(np.array([[1.0, 2.0, 0.5],
                                   [0.0, 1.0, 1.0],
                                   [-1.0, 3.0, 0.0],
                                   [2.0, -2.0, 1.0]], dtype=np.float32))
    x = np.array([[inf, 1.0, 2.0],
                  [inf, -inf, 1.0],
                  [nan, 1.0, 1.0],
                  [1.0, 2.0, 3.0]], dtype=np.float32)
    y, s = gemv_rows(w, x)
    want = np.array([[inf, nan, -inf, inf],     # inf+2+1, 0*inf, -inf+3, 2inf-2+2
                     [nan, nan, -inf, inf],     # inf-2inf, 0*inf, -inf-3inf, 2inf+2inf+1
                     [nan, nan, nan, nan],
                     [6.5, 5.0, 5.0, 1.0]])
    np.testing.assert_array_equal(y, want)
    assert np.isinf(s[0, 0]) and np.isnan(s[0, 1]) and s[3, 3] == 2 + 4 + 3


def test_subnormal_activations_are_ordinary_values():
    w = f32_to_bf16_bits(np.array([[1.0, 2.0, 1.0]], dtype=np.float32))
    x = np.array([[2.0 ** -130, 2.0 ** -140, 0.0]], dtype=np.float32)
    y, _ = gemv_rows(w, x)
    assert y[0, 0] == 2.0 ** -130 + 2.0 ** -139
