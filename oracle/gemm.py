"""Block-scaled FP8 GEMM reference (oracle; test infrastructure only).

What is computed [paperlayer.ai summary, appendix C "Production Training
Details", bullet "FP8 implementation pipeline": forward, data-gradient and
weight-gradient GEMMs of the linear layers take blockwise E4M3 operands;
paper.rainbus.top summary, 方法步骤详情 step (3): Fprop/Dgrad/Wgrad all in E4M3]:

    D[i, j] = sum_k deq(A)[i, k] * deq(B)[j, k],   deq(q) = 2^e * decode(q)

with A grouped 1x128 along k and B either 128x128-tiled (fprop, dgrad) or
1x128-grouped along k (wgrad). Reading: the reference value is this sum
taken exactly on the dequantised operands. Within one 128-block the products of
two E4M3 values share the factor 2^(ea+eb) and are integer multiples of
2^-18 * 2^(ea+eb) below 2^18, so a float64 sum of 128 of them is exact; only the
cross-block additions round, at the 2^-53 level. A float64 matmul of the exactly
dequantised operands is therefore this definition up to that rounding.

The fast path accumulates in FP32 and writes BF16 (the pages do not fix the
accumulator; FP32 accumulation and BF16 output are the readings taken). It is
judged per element against the unrounded float64 value:
    |gpu - ref| <= 2^-7 * |ref| + 1e-3 * rms(ref).

A second, always-applicable bound (contract_allowance) states what FP32
accumulation delivers on a matrix unit that adds the products of each aligned
group of 8 consecutive k in a fixed-point window: every product is truncated
toward zero to a multiple of 2^(E-13), E = floor(log2) of the group's largest
product magnitude, and the group sums are accumulated in FP32. Each group then
loses less than 7 * 2^(E-13) <= 7 * 2^-13 * max_g |a b|, each FP32 rounding
of a running sum at most 2^-24 of its magnitude (there are fewer than K/4 of
them: K/8 group sums, plus one scale FMA per 128-block where the scales are
applied outside the matrix instruction), and the BF16 output rounding at most
2^-8 of the value:
    |gpu - ref| <= 2^-8 |ref|
                   + (1 + 2^-8) * (7 * 2^-13 * sum_g max_{k in g} |a_k b_k|
                                   + (K/4) * 2^-24 * sum_k |a_k b_k|).
It is a statement about the accumulator, not about the method: the method is
the exact sum above.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict

import numpy as np

from .e4m3 import decode_e4m3

GROUP = 128
WINDOW_GROUP = 8  # products summed together in one fixed-point window


def dequant_act_groups(q: np.ndarray, dscale: np.ndarray) -> np.ndarray:
    """Dequantise reduction-contiguous codes q [rows, K] whose scales are dscale [K/128, rows]."""
    rows, k = q.shape
    if dscale.shape[0] != k // GROUP or dscale.shape[1] < rows:
        raise ValueError("dscale shape does not match codes")
    s = np.repeat(dscale[:, :rows].astype(np.float64).T, GROUP, axis=1)  # [rows, K]
    return decode_e4m3(q) * s


def dequant_w_tiles(q: np.ndarray, dscale_tiles: np.ndarray) -> np.ndarray:
    """Dequantise codes q [R, C] whose scales are one per 128x128 tile, dscale_tiles [R/128, C/128]."""
    r, c = q.shape
    s = np.repeat(np.repeat(dscale_tiles.astype(np.float64), GROUP, axis=0), GROUP, axis=1)
    return decode_e4m3(q) * s[:r, :c]


def gemm_fprop(qx, sx, qw, sw) -> np.ndarray:
    """Y[M, N] = deq(X)[M, K] . deq(W)[N, K]^T.  qx [M,K], sx [K/128, M]; qw [N,K], sw [N/128, K/128]."""
    return dequant_act_groups(qx, sx) @ dequant_w_tiles(qw, sw).T


def gemm_dgrad(qdy, sdy, qwt, sw) -> np.ndarray:
    """dX[M, Kw] = deq(dY)[M, Nw] . deq(W)[Nw, Kw].

    qdy [M, Nw] with sdy [Nw/128, M] (groups along Nw); qwt = W's codes transposed
    [Kw, Nw]; sw = W's tile grid [Nw/128, Kw/128] (so Wt's tile (a, b) has scale sw[b, a]).
    """
    return dequant_act_groups(qdy, sdy) @ dequant_w_tiles(qwt, sw.T).T


def gemm_wgrad(qdyt, sdy, qxt, sx) -> np.ndarray:
    """dW[Nw, Kw] = deq(dY)^T . deq(X), both grouped along the token dimension M.

    qdyt [Nw, M] with sdy [M/128, Nw]; qxt [Kw, M] with sx [M/128, Kw].
    """
    return dequant_act_groups(qdyt, sdy) @ dequant_act_groups(qxt, sx).T


def gemm_blockwise_exact(qa, sa_rows, qb, sb_rows) -> list:
    """Second path for tiny sizes: exact rationals, scale applied per 128-block.

    qa [m, K] codes; sa_rows[kb][i] is the multiplier of A's row i in K-block kb;
    likewise sb_rows[kb][j] for B's row j (callers expand tile scales per row).
    Returns a list of lists of Fractions: sum_kb sa*sb * (sum_{k in kb} qa*qb).
    """
    m, k = qa.shape
    n = qb.shape[0]
    va = decode_e4m3(qa)
    vb = decode_e4m3(qb)
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            total = Fraction(0)
            for kb in range(k // GROUP):
                part = Fraction(0)
                for kk in range(kb * GROUP, (kb + 1) * GROUP):
                    part += Fraction(float(va[i, kk])) * Fraction(float(vb[j, kk]))
                total += Fraction(float(sa_rows[kb][i])) * Fraction(float(sb_rows[kb][j])) * part
            row.append(total)
        out.append(row)
    return out


def unquantized_reference(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """float64 A . B^T of the bf16 inputs, without quantisation: the sanity reference for the
    quantisation error, and the definition the plain BF16 comparison GEMM is checked against
    (products of two bf16 values are exact in float64; only the additions round, at 2^-53)."""
    def f64(bits):
        return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return f64(a_bits) @ f64(b_bits).T


def bf16_round_from_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one rounding, nearest-even (finite, in bf16 range)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    bits = x.view(np.uint64) if x.flags.c_contiguous else np.ascontiguousarray(x).view(np.uint64)
    # normal bf16 range: keep 7 of the 52 fraction bits, round half to even
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rnd = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    y = rnd.view(np.float64)
    # bf16 subnormals (|x| < 2^-126): quantum 2^-133
    small = a < 2.0 ** -126
    y = np.where(small, np.copysign(np.rint(a * 2.0 ** 133) * 2.0 ** -133, x), y)
    if np.any(np.abs(y) > 3.3895313892515355e38):
        raise ValueError("bf16_round_from_f64: out of bf16 range")
    f32 = y.astype(np.float32)  # exact: y has at most 8 significant bits
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def gemm_tolerance_report(gpu: np.ndarray, ref64: np.ndarray) -> Dict[str, float]:
    """Per-element bound |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), plus diagnostics."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref64 * ref64))) if ref64.size else 0.0
    bound = 2.0 ** -7 * np.abs(ref64) + 1e-3 * rms
    err = np.abs(gpu - ref64)
    viol = int(np.count_nonzero(~(err <= bound)))
    ratio = float(np.max(err / np.where(bound > 0, bound, 1.0))) if err.size else 0.0
    ref_bf16 = bf16_round_from_f64(ref64)
    gpu_bits = (gpu.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return {
        "violations": viol,
        "max_err_over_bound": ratio,
        "rms_ref": rms,
        "frac_bit_equal_bf16": float(np.mean(gpu_bits == ref_bf16)) if gpu.size else 1.0,
        "n": int(gpu.size),
    }


def contract_allowance(a_deq: np.ndarray, b_deq: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    """Per-element allowance of the accumulation contract (module docstring) for
    D[i, j] = sum_k a_deq[i, k] * b_deq[j, k], given the exact ref64 = that sum.

    a_deq [m, K], b_deq [n, K] are the dequantised operands (float64); K % 8 == 0."""
    a = np.abs(np.asarray(a_deq, dtype=np.float64))
    b = np.abs(np.asarray(b_deq, dtype=np.float64))
    m, k = a.shape
    if b.shape[1] != k or k % WINDOW_GROUP:
        raise ValueError("operands must share a K that is a multiple of 8")
    abs_sum = a @ b.T
    group_max_sum = np.zeros((m, b.shape[0]))
    for g in range(0, k, WINDOW_GROUP):
        gmax = np.zeros((m, b.shape[0]))
        for kk in range(g, g + WINDOW_GROUP):
            np.maximum(gmax, np.multiply.outer(a[:, kk], b[:, kk]), out=gmax)
        group_max_sum += gmax
    window = 7.0 * 2.0 ** -13 * group_max_sum + (k // 4) * 2.0 ** -24 * abs_sum
    return 2.0 ** -8 * np.abs(np.asarray(ref64, dtype=np.float64)) + (1.0 + 2.0 ** -8) * window


def contract_report(gpu: np.ndarray, ref64: np.ndarray, allowance: np.ndarray) -> Dict[str, float]:
    """Elements outside the accumulation contract's allowance, and the worst error / allowance."""
    err = np.abs(np.asarray(gpu, dtype=np.float64) - np.asarray(ref64, dtype=np.float64))
    allowance = np.asarray(allowance, dtype=np.float64)
    viol = int(np.count_nonzero(~(err <= allowance)))
    ratio = float(np.max(err / np.where(allowance > 0, allowance, 1.0))) if err.size else 0.0
    return {"violations": viol, "max_err_over_allowance": ratio, "n": int(err.size)}
