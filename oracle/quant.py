"""Online block quantisers (oracle; test infrastructure only).

What is computed [paper.rainbus.top summary, 前置知识 "FP8 块级混合精度训练" and
方法步骤详情 step (3); ta-paperlens explainer, 打ち手2 (report §3.2)]:
activations and gradients are split into groups of 128 consecutive values
along the GEMM reduction dimension, weights into aligned 128x128 tiles; each
group gets its own power-of-two scale, computed from that group alone when the
tensor is quantised, and every value is stored as an E4M3 code.

Step order, for every group G:
  1. amax(G) = max |x| over the group (exact);
  2. e(G) = the smallest integer with amax <= 448 * 2^e (reading: the largest
     scale-down that never saturates, so a block's maximum maps to at most 448);
     e = 0 for an all-zero group; e >= -126 (2^e is then an fp32 normal);
  3. q = E4M3 code of x * 2^-e (exact in float64), rounded to nearest-even;
  4. the dequantisation multiplier s = 2^e is returned as float32.

Inputs are bf16 bit patterns (uint16). Outputs follow the C-ABI layouts:
  row mode  (groups along columns): q [R, C],        dscale [C/128][R]
  col mode  (groups along rows):    q [C, R] (transposed), dscale [R/128][C]
  weights   (128x128 tiles):        q [N, K], qt [K, N], dscale [N/128][K/128]
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .e4m3 import encode_e4m3

GROUP = 128
E_MIN = -126


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, for amax >= 0 (float64, exact).

    Write amax = f * 2^x with f in [0.5, 1) (frexp, exact). Since 448 = 0.875 * 2^9,
    amax <= 448 * 2^e  <=>  f * 2^(x - e) <= 0.875 * 2^9, which holds for
    e >= x - 9 when f <= 0.875 and for e >= x - 8 when f > 0.875.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(amax < 0) or not np.all(np.isfinite(amax)):
        raise ValueError("block_exponent: amax must be finite and >= 0")
    f, x = np.frexp(amax)
    e = x.astype(np.int64) - 9 + (f > 0.875).astype(np.int64)
    e = np.where(amax == 0.0, 0, e)
    return np.maximum(e, E_MIN)


def _quantise_groups(xg: np.ndarray, axes) -> Tuple[np.ndarray, np.ndarray]:
    amax = np.abs(xg).max(axis=axes, keepdims=True)
    e = block_exponent(amax)
    codes = encode_e4m3(np.ldexp(xg, -e))
    return codes, e


def quant_act_1x128(x_bits: np.ndarray, along: str = "cols") -> Tuple[np.ndarray, np.ndarray]:
    """1x128 activation/gradient quantiser.

    along="cols": groups are 128 consecutive elements of a row (row mode; fprop X
    along K, dgrad dY along N). Returns q uint8 [R, C] and dscale float32 [C/128, R].
    along="rows": groups are 128 consecutive rows of a column (col mode; wgrad dY and
    X along tokens). Returns q uint8 [C, R] (reduction dim contiguous) and dscale
    float32 [R/128, C].
    """
    x = _bf16_to_f64(x_bits)
    if x.ndim != 2:
        raise ValueError("expected a 2-D tensor")
    rows, cols = x.shape
    if along == "cols":
        if cols % GROUP:
            raise ValueError("cols must be a multiple of 128")
        xg = x.reshape(rows, cols // GROUP, GROUP)
        codes, e = _quantise_groups(xg, axes=2)
        q = codes.reshape(rows, cols)
        dscale = np.ldexp(1.0, e[:, :, 0]).astype(np.float32).T.copy()
        return q, dscale
    if along == "rows":
        if rows % GROUP:
            raise ValueError("rows must be a multiple of 128")
        xg = x.reshape(rows // GROUP, GROUP, cols)
        codes, e = _quantise_groups(xg, axes=1)
        q = codes.reshape(rows, cols).T.copy()
        dscale = np.ldexp(1.0, e[:, 0, :]).astype(np.float32)
        return q, dscale
    raise ValueError(f"along must be 'cols' or 'rows', got {along!r}")


def quant_w_128x128(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """128x128 weight-tile quantiser.

    Returns q uint8 [N, K], qt uint8 [K, N] (the same codes transposed, used by
    the data-gradient GEMM) and dscale float32 [N/128, K/128].
    """
    w = _bf16_to_f64(w_bits)
    n, k = w.shape
    if n % GROUP or k % GROUP:
        raise ValueError("weight dims must be multiples of 128")
    wg = w.reshape(n // GROUP, GROUP, k // GROUP, GROUP)
    codes, e = _quantise_groups(wg, axes=(1, 3))
    q = codes.reshape(n, k)
    dscale = np.ldexp(1.0, e[:, 0, :, 0]).astype(np.float32)
    return q, q.T.copy(), dscale
