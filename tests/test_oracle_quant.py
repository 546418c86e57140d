"""Pins for the oracle's block quantisers (CPU only).

Grouping and layout are checked against scalar Python loops on tiny tensors,
the codes against hand-derived worked examples (tests/golden/), and the whole
against invariants the method implies.
"""
import bisect
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import decode_e4m3, quant_act_1x128, quant_w_128x128
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _parse(s: str) -> float:
    if "p" in s:
        mant, exp = s.split("p")
        return math.ldexp(float(mant), int(exp))
    return float(s)


def _bits(vals) -> np.ndarray:
    f = np.array(vals, dtype=np.float32)
    b = f32_to_bf16_bits(f)
    assert np.array_equal(bf16_bits_to_f32(b), f), "worked example values must be exact bf16"
    return b


# ---- scalar reference pieces, written independently of the oracle -----------------------------

_MAGS = sorted({float(Fraction(m, 8) * Fraction(2) ** -6) for m in range(8)}
               | {float((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)) for e in range(1, 16) for m in range(8)
                  if not (e == 15 and m == 7)})
_MAG_CODE = {}
for _e in range(16):
    for _m in range(8):
        if _e == 15 and _m == 7:
            continue
        _v = float(Fraction(_m, 8) * Fraction(2) ** -6) if _e == 0 else float((1 + Fraction(_m, 8)) * Fraction(2) ** (_e - 7))
        _MAG_CODE[_v] = (_e << 3) | _m


def _scalar_code(x: float) -> int:
    a = abs(x)
    i = bisect.bisect_left(_MAGS, a)
    cands = [c for c in (i - 1, i) if 0 <= c < len(_MAGS)]
    best = min(cands, key=lambda c: (abs(_MAGS[c] - a), _MAG_CODE[_MAGS[c]] & 1))
    code = _MAG_CODE[_MAGS[best]]
    return code | (0x80 if math.copysign(1.0, x) < 0 else 0)


def _scalar_e(amax: float) -> int:
    if amax == 0.0:
        return 0
    e = -200
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return max(e, -126)


def _scalar_quant_group(vals):
    amax = max(abs(v) for v in vals)
    e = _scalar_e(amax)
    return [_scalar_code(v * 2.0 ** -e) for v in vals], e


# ---- grouping / layout by brute force --------------------------------------------------------

def _rand_bits(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    # sprinkle zeros, negative zeros, outliers and tiny values
    flat = x.reshape(-1)
    flat[rng.choice(flat.size, 7, replace=False)] = 0.0
    flat[rng.choice(flat.size, 5, replace=False)] = -0.0
    flat[rng.choice(flat.size, 5, replace=False)] *= 50
    flat[rng.choice(flat.size, 5, replace=False)] *= 1e-30
    return f32_to_bf16_bits(x)


def test_row_mode_matches_scalar_loops():
    bits = _rand_bits((3, 384), 1)
    x = bf16_bits_to_f32(bits).astype(np.float64)
    q, s = quant_act_1x128(bits, "cols")
    assert q.shape == (3, 384) and s.shape == (3, 3) and q.dtype == np.uint8 and s.dtype == np.float32
    for r in range(3):
        for g in range(3):
            codes, e = _scalar_quant_group([float(v) for v in x[r, 128 * g:128 * g + 128]])
            assert list(q[r, 128 * g:128 * g + 128]) == codes
            assert s[g, r] == 2.0 ** e


def test_col_mode_matches_scalar_loops():
    bits = _rand_bits((256, 5), 2)
    x = bf16_bits_to_f32(bits).astype(np.float64)
    q, s = quant_act_1x128(bits, "rows")
    assert q.shape == (5, 256) and s.shape == (2, 5)
    for c in range(5):
        for g in range(2):
            codes, e = _scalar_quant_group([float(v) for v in x[128 * g:128 * g + 128, c]])
            assert list(q[c, 128 * g:128 * g + 128]) == codes
            assert s[g, c] == 2.0 ** e


def test_weight_tiles_match_scalar_loops():
    bits = _rand_bits((256, 128), 3, 0.02)
    x = bf16_bits_to_f32(bits).astype(np.float64)
    q, qt, s = quant_w_128x128(bits)
    assert q.shape == (256, 128) and qt.shape == (128, 256) and s.shape == (2, 1)
    assert np.array_equal(qt, q.T)
    for tb in range(2):
        tile = x[128 * tb:128 * tb + 128, :]
        codes, e = _scalar_quant_group([float(v) for v in tile.reshape(-1)])
        assert list(q[128 * tb:128 * tb + 128, :].reshape(-1)) == codes
        assert s[tb, 0] == 2.0 ** e


# ---- hand-derived worked examples -----------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("idx", range(7))
def test_worked_example_row_groups(idx):
    ex = _golden()["row_groups"][idx]
    vals = [_parse(v) for v in ex["values"]]
    row = vals + [0.0] * (128 - len(vals))
    q, s = quant_act_1x128(_bits([row]), "cols")
    assert s[0, 0] == 2.0 ** ex["e"]
    assert [f"{c:02X}" for c in q[0, :len(vals)]] == ex["codes"]
    # the same group as a column (col mode) gives the same codes and scale
    qc, sc = quant_act_1x128(_bits(np.array([row]).T), "rows")
    assert sc[0, 0] == 2.0 ** ex["e"]
    assert [f"{c:02X}" for c in qc[0, :len(vals)]] == ex["codes"]


def test_worked_example_weight_tile():
    ex = _golden()["weight_tile"]
    w = np.zeros((128, 128), dtype=np.float32)
    for r, c, v, _ in ex["entries"]:
        w[r, c] = _parse(v)
    q, qt, s = quant_w_128x128(_bits(w))
    assert s[0, 0] == 2.0 ** ex["e"]
    for r, c, _, code in ex["entries"]:
        assert f"{q[r, c]:02X}" == code
        assert f"{qt[c, r]:02X}" == code


# ---- invariants ------------------------------------------------------------------------------

def _mixed_bits(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, size=(rows, 1))).astype(np.float32)  # wide per-row dynamic range
    x.reshape(-1)[rng.choice(x.size, x.size // 50, replace=False)] *= 50
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("along", ["cols", "rows"])
def test_scales_are_powers_of_two_and_block_max_lands_in_top_binade(along):
    bits = _mixed_bits(256, 384, 4)
    x = bf16_bits_to_f32(bits).astype(np.float64)
    q, s = quant_act_1x128(bits, along)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5), "every scale is an exact power of two"
    deq = decode_e4m3(q)
    if along == "cols":
        amax = np.abs(x.reshape(256, 3, 128)).max(-1).T  # [3, 256]
        code_max = np.abs(deq.reshape(256, 3, 128)).max(-1).T
    else:
        amax = np.abs(x.reshape(2, 128, 384)).max(1)  # [2, 384]
        code_max = np.abs(deq.reshape(384, 2, 128)).max(-1).T
    ratio = amax / s
    nz = amax > 0
    assert np.all(ratio[nz] <= 448.0) and np.all(ratio[nz] > 224.0)
    # the block maximum's code has exponent field 14 or 15, i.e. lies in [224, 448]
    assert np.all((code_max[nz] >= 224.0) & (code_max[nz] <= 448.0))


def test_scale_equivariance_and_sign_symmetry():
    bits = _mixed_bits(128, 256, 5)
    x = bf16_bits_to_f32(bits)
    q0, s0 = quant_act_1x128(bits, "cols")
    for t in (-5, 3, 11):
        q1, s1 = quant_act_1x128(f32_to_bf16_bits(x * np.float32(2.0 ** t)), "cols")
        assert np.array_equal(q1, q0)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** t)
    qn, sn = quant_act_1x128(f32_to_bf16_bits(-x), "cols")
    assert np.array_equal(qn, q0 ^ 0x80)
    assert np.array_equal(sn, s0)


def test_exactly_representable_values_round_trip():
    rng = np.random.default_rng(6)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = decode_e4m3(codes)
    for j in (-9, 0, 4):
        blk = rng.choice(vals, size=(4, 128))
        # pin each block's maximum inside (224, 448] so that its scale is exactly 2^j
        blk[:, 0] = rng.choice([-448.0, -256.0, 240.0, 448.0], size=4)
        x = (blk * 2.0 ** j).astype(np.float32)
        q, s = quant_act_1x128(f32_to_bf16_bits(x), "cols")
        assert np.all(s == 2.0 ** j)
        assert np.array_equal(decode_e4m3(q) * s[0][:, None], x.astype(np.float64))


def test_block_locality():
    bits = _mixed_bits(256, 256, 7)
    q0, s0 = quant_act_1x128(bits, "cols")
    qw0, _, sw0 = quant_w_128x128(bits)
    b2 = bits.copy()
    b2[130, 5] = f32_to_bf16_bits(np.array([1e35], dtype=np.float32))[0]
    q1, s1 = quant_act_1x128(b2, "cols")
    changed = np.argwhere(q1 != q0)
    assert set(map(tuple, np.unique(np.stack([changed[:, 0], changed[:, 1] // 128], 1), axis=0))) == {(130, 0)}
    assert np.argwhere(s1 != s0).tolist() == [[0, 130]]
    qw1, _, sw1 = quant_w_128x128(b2)
    ch = np.argwhere(qw1 != qw0)
    assert np.all(ch[:, 0] // 128 == 1) and np.all(ch[:, 1] // 128 == 0)
    assert np.argwhere(sw1 != sw0).tolist() == [[1, 0]]


def test_weight_retile_equals_transpose():
    bits = _mixed_bits(256, 384, 8)
    q, qt, s = quant_w_128x128(bits)
    q2, qt2, s2 = quant_w_128x128(np.ascontiguousarray(bits.T))
    assert np.array_equal(q2, qt) and np.array_equal(qt2, q) and np.array_equal(s2, s.T)


def test_shape_errors():
    with pytest.raises(ValueError):
        quant_act_1x128(np.zeros((4, 100), np.uint16), "cols")
    with pytest.raises(ValueError):
        quant_act_1x128(np.zeros((100, 4), np.uint16), "rows")
    with pytest.raises(ValueError):
        quant_w_128x128(np.zeros((128, 200), np.uint16))
