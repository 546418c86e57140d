"""Pins for the oracle's E4M3 codec and exponent rule (CPU only).

Each check compares the oracle with something that is not the oracle: the bit
layout's closed-form values, a brute-force nearest-code search, exact
rationals, and torch's own float8_e4m3fn cast as a library special case.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import block_exponent, decode_e4m3, encode_e4m3, e4m3_table


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    return vals[np.isfinite(vals)].astype(np.float64)


def _brute_force_nearest(v):
    """Nearest finite E4M3 code by exhaustive search over the 127 magnitudes; ties -> even code."""
    mags = np.array([float(Fraction(m, 8) * Fraction(2) ** -6) for m in range(8)]
                    + [float((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)) for e in range(1, 16) for m in range(8)
                       if not (e == 15 and m == 7)])
    codes = np.arange(127)
    a = np.abs(v)[:, None]
    d = np.abs(a - mags[None, :])  # exact in float64: both sides have few significant bits
    best = d.min(axis=1, keepdims=True)
    tied = d == best
    # among tied codes prefer the even one (the two neighbours of a midpoint differ in the last bit)
    even_pref = np.where(tied & (codes[None, :] % 2 == 0), codes[None, :], 1000).min(axis=1)
    any_pref = np.where(tied, codes[None, :], 1000).min(axis=1)
    code = np.where(even_pref < 1000, even_pref, any_pref)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_decode_closed_form_values():
    t = e4m3_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x44] == 3.0
    assert t[0x78] == 256.0 and t[0x76] == 224.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.count_nonzero(np.isnan(t)) == 2
    # every finite code decodes to a distinct value (apart from the two zeros)
    fin = t[np.isfinite(t)]
    assert len(np.unique(fin)) == 253


def test_encode_decode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_encode_matches_brute_force_on_every_bf16_value():
    v = _all_bf16_values()
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(encode_e4m3(v), _brute_force_nearest(v))


def test_encode_matches_brute_force_on_scaled_significands():
    # every bf16 significand at every exponent from 2^-40 to 2^8 (covers x * 2^-e for any block)
    sig = 1.0 + np.arange(128) / 128.0
    v = np.concatenate([np.ldexp(sig, e) for e in range(-40, 9)])
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(encode_e4m3(v), _brute_force_nearest(v))


def test_encode_midpoints_round_half_to_even():
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80),
             (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02), (7 * 2.0 ** -10, 0x04), (448.0, 0x7E),
             (15 * 2.0 ** -10, 0x08), (0.0, 0x00), (-0.0, 0x80), (232.0, 0x76), (248.0, 0x78)]
    for v, c in cases:
        assert encode_e4m3(np.array([v]))[0] == c, v


def test_encode_agrees_with_torch_float8_cast():
    v = _all_bf16_values()
    v = v[np.abs(v) <= 448.0]
    t = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3(v), t)


def test_encode_rejects_out_of_range_and_nonfinite():
    with pytest.raises(ValueError):
        encode_e4m3(np.array([449.0]))
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.nan]))


def _smallest_e_exact(amax: Fraction) -> int:
    """Definition: the smallest integer e with amax <= 448 * 2^e (search by exact rationals)."""
    e = 0
    two = Fraction(2)
    while amax <= 448 * two ** (e - 1):
        e -= 1
    while amax > 448 * two ** e:
        e += 1
    return e


def test_exponent_rule_exhaustive_over_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)  # every positive finite bf16
    vals = (bits << 16).view(np.float32).astype(np.float64)
    got = block_exponent(vals)
    want = np.array([max(_smallest_e_exact(Fraction(float(x))), -126) for x in vals])
    assert len(vals) == 32639
    assert np.array_equal(got, want)


def test_exponent_rule_zero_block_and_clamp():
    assert block_exponent(np.array([0.0]))[0] == 0
    assert block_exponent(np.array([2.0 ** -133]))[0] == -126
    assert block_exponent(np.array([448.0 * 2.0 ** -126]))[0] == -126
    assert block_exponent(np.array([448.0 * 2.0 ** -127]))[0] == -126
    # the largest bf16 needs e = 120, far from any upper limit
    big = float((np.array([0x7F7F << 16], dtype=np.uint32)).view(np.float32)[0])
    assert block_exponent(np.array([big]))[0] == 120
