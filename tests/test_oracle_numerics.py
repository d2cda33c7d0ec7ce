"""Pins of the oracle's exact input conversions (oracle/numerics.py).

Every bf16 parity claim goes through ``bf16_bits_to_f64``, so it is pinned
here against what the formats fix, independently of its own arithmetic:

* bfloat16 is the upper half of an IEEE 754 binary32 (1 sign bit, 8
  exponent bits with bias 127, 7 fraction bits); hand-decoded patterns
  below follow that definition (normal, subnormal, signed zero, infinities,
  NaN, largest finite);
* every one of the 65,536 bit patterns agrees with torch's own bfloat16 ->
  float64 conversion (a library routine that shares nothing with the
  oracle), NaN for NaN;
* the float64 value, rounded back to bfloat16 by torch, gives the same bits
  (round trip on every non-NaN pattern).
"""

import math

import numpy as np
import torch

from oracle.numerics import bf16_bits_to_f64, exact_column_sums, f32_to_f64


def _decode_bf16(bits: int) -> float:
    """Value of a bfloat16 pattern from the field definition (sign, 8-bit
    biased exponent, 7-bit fraction), in exact binary arithmetic."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


HAND = [
    (0x3F80, 1.0),
    (0xC040, -3.0),
    (0x4049, 3.140625),                 # 1.5703125 * 2
    (0x3E80, 0.25),
    (0x0080, 2.0 ** -126),              # smallest normal
    (0x0001, 2.0 ** -133),              # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),        # largest subnormal
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def test_hand_decoded_patterns():
    bits = np.array([b for b, _ in HAND], dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    for (b, want), g in zip(HAND, got):
        assert g == want, "0x%04X: %r != %r" % (b, g, want)
        assert _decode_bf16(b) == want


def test_signed_zero_and_nan():
    got = bf16_bits_to_f64(np.array([0x0000, 0x8000, 0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))
    assert got[0] == 0.0 and not math.copysign(1.0, got[0]) < 0
    assert got[1] == 0.0 and math.copysign(1.0, got[1]) < 0
    assert np.all(np.isnan(got[2:]))


def test_all_patterns_match_field_decoding_and_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = bf16_bits_to_f64(bits)
    # the same patterns as signed 16-bit (the form the tests pass from torch)
    got_signed = bf16_bits_to_f64(bits.view(np.int16))
    assert np.array_equal(got, got_signed, equal_nan=True)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, lib, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(lib))
    ref = np.array([_decode_bf16(int(b)) for b in bits], dtype=np.float64)
    assert np.array_equal(got, ref, equal_nan=True)
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_round_trip_through_torch_rounding():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    finite = ~np.isnan(vals)
    back = torch.from_numpy(vals[finite]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(back, bits[finite])


def test_f32_to_f64_exact():
    x = np.array([0.1, -2.5, 1e-45, 3.4028234663852886e38], dtype=np.float32)
    got = f32_to_f64(x)
    # 0.1f is 13421773 * 2^-27 exactly; 1e-45f is the smallest subnormal 2^-149
    assert got[0] == 13421773 * 2.0 ** -27
    assert got[1] == -2.5
    assert got[2] == 2.0 ** -149
    assert got[3] == (2 - 2.0 ** -23) * 2.0 ** 127
    assert np.array_equal(got.astype(np.float32), x)


# ------------------------------------------------------ exact column sums

def _fsum_cols(x):
    return np.array([math.fsum(x[:, c].tolist()) for c in range(x.shape[1])])


def test_exact_column_sums_fixes_what_plain_summation_rounds():
    # 2^60 + 1 rounds to 2^60 in float64: a plain left-to-right sum gives 0
    x = np.array([[2.0 ** 60], [1.0], [-(2.0 ** 60)]])
    assert x.sum(axis=0)[0] == 0.0
    assert exact_column_sums(x)[0] == 1.0
    # a tie: 1 + 2^-53 is halfway between 1 and 1 + 2^-52 and rounds to even
    y = np.array([[1.0], [2.0 ** -54], [2.0 ** -54]])
    assert exact_column_sums(y)[0] == 1.0
    z = np.array([[1.0], [2.0 ** -53], [2.0 ** -60]])
    assert exact_column_sums(z)[0] == 1.0 + 2.0 ** -52


def test_exact_column_sums_match_fsum_on_mixed_magnitudes():
    rng = np.random.default_rng(5)
    for span in (8, 30, 45, 60, 74, 100, 140):
        for n in (1, 2, 7, 64, 128):
            mag = 2.0 ** rng.uniform(-span / 2, span / 2, (n, 24))
            x = (mag * rng.choice([-1.0, 1.0], (n, 24))).astype(np.float32).astype(np.float64)
            if n > 2:
                x[1] = -x[0]                      # cancellation
                x[2, ::3] = 0.0                   # zeros
            assert np.array_equal(exact_column_sums(x), _fsum_cols(x)), (span, n)


def test_exact_column_sums_certified_columns_and_edge_values():
    rng = np.random.default_rng(6)
    # ordinary bf16-like data: every column certified, numpy's sum already exact
    bits = (rng.standard_normal((128, 32)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = bf16_bits_to_f64(bits)
    assert np.array_equal(exact_column_sums(x), _fsum_cols(x))
    # subnormal and huge binary32 values, all-zero columns, one row, no rows
    e = np.array([[1e-45, 3.4e38, 0.0], [-1e-45, -3.4e38, 0.0], [2e-45, 1.0, 0.0]], dtype=np.float32)
    e = e.astype(np.float64)
    assert np.array_equal(exact_column_sums(e), _fsum_cols(e))
    assert np.array_equal(exact_column_sums(e[:1]), e[0])
    assert exact_column_sums(np.zeros((0, 3))).shape == (3,)
