"""Pins for the oracle's block-scaled GEMM (CPU only).

Exact rational sums on tiny shapes, closed forms (identity, one-hot,
permutation and power-of-two-scaled weights), a hand-derived worked example,
and the sanity bound on quantisation error against the unquantised product.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (
    bf16_round_from_f64,
    decode_e4m3,
    gemm_blockwise_exact,
    gemm_dgrad,
    gemm_fprop,
    gemm_tolerance_report,
    gemm_wgrad,
    quant_act_1x128,
    quant_w_128x128,
    unquantized_reference,
)
from workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _rand(shape, seed, sigma=1.0, outliers=0.01):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    x.reshape(-1)[rng.choice(x.size, max(1, int(outliers * x.size)), replace=False)] *= 50
    return _bits(x)


def _close_to_exact(got, exact_rows, k):
    for i, row in enumerate(exact_rows):
        for j, ex in enumerate(row):
            tol = Fraction(k // 128) * Fraction(2) ** -52 * (abs(ex) + 1)
            assert abs(Fraction(float(got[i, j])) - ex) <= tol * 4, (i, j)


@pytest.mark.parametrize("k", [128, 256, 512])
def test_fprop_matches_exact_rational_block_sums(k):
    xb, wb = _rand((5, k), 10 + k), _rand((128, k), 20 + k, 0.02)
    qx, sx = quant_act_1x128(xb, "cols")
    qw, _, sw = quant_w_128x128(wb)
    y = gemm_fprop(qx, sx, qw, sw)
    sb_rows = [[sw[j // 128, kb] for j in range(128)] for kb in range(k // 128)]
    exact = gemm_blockwise_exact(qx, sx, qw[:7], [r[:7] for r in sb_rows])
    _close_to_exact(y[:, :7], exact, k)


def test_dgrad_and_wgrad_match_exact_rational_block_sums():
    # dgrad: dX[M, Kw] = dY[M, Nw] . W[Nw, Kw], dY grouped along Nw, W tiles read transposed
    dyb, wb = _rand((4, 256), 31, 1e-3), _rand((256, 128), 32, 0.01)
    qdy, sdy = quant_act_1x128(dyb, "cols")
    qw, qwt, sw = quant_w_128x128(wb)
    dx = gemm_dgrad(qdy, sdy, qwt, sw)
    assert dx.shape == (4, 128)
    sb_rows = [[sw[kb, j // 128] for j in range(128)] for kb in range(2)]
    exact = gemm_blockwise_exact(qdy, sdy, qwt[:6], [r[:6] for r in sb_rows])
    _close_to_exact(dx[:, :6], exact, 256)
    # wgrad: dW[Nw, Kw] = dY^T . X, both grouped along 256 tokens
    dyb, xb = _rand((256, 6), 33, 1e-3), _rand((256, 5), 34)
    qdyt, sdy = quant_act_1x128(dyb, "rows")
    qxt, sx = quant_act_1x128(xb, "rows")
    dw = gemm_wgrad(qdyt, sdy, qxt, sx)
    assert dw.shape == (6, 5)
    exact = gemm_blockwise_exact(qdyt, sdy, qxt, sx)
    _close_to_exact(dw, exact, 256)


def test_layouts_agree_with_plain_definition_on_dequantised_operands():
    # the three layouts all compute sum_k deq(A)[i,k] deq(B)[j,k]; check against dense loops
    xb, wb = _rand((3, 256), 40), _rand((128, 256), 41, 0.02)
    qx, sx = quant_act_1x128(xb, "cols")
    qw, qwt, sw = quant_w_128x128(wb)
    dx = decode_e4m3(qx) * np.repeat(sx.T.astype(np.float64), 128, 1)
    dw = decode_e4m3(qw) * np.kron(sw.astype(np.float64), np.ones((128, 128)))
    y = gemm_fprop(qx, sx, qw, sw)
    for i in range(3):
        for j in range(0, 128, 17):
            assert y[i, j] == pytest.approx(sum(dx[i, k] * dw[j, k] for k in range(256)), rel=1e-14, abs=1e-300)


def test_identity_weight_reproduces_dequantised_input_bit_exactly():
    xb = _rand((64, 256), 50)
    qx, sx = quant_act_1x128(xb, "cols")
    eye = np.eye(256, dtype=np.float32)
    qw, qwt, sw = quant_w_128x128(_bits(eye))
    # diagonal tiles: amax 1 -> e = -8, diagonal code 0x78 (256); off-diagonal tiles all zero -> e = 0
    assert np.array_equal(sw, np.array([[2.0 ** -8, 1.0], [1.0, 2.0 ** -8]], dtype=np.float32))
    assert np.all(np.diag(qw) == 0x78) and np.count_nonzero(qw) == 256
    y = gemm_fprop(qx, sx, qw, sw)
    deq_x = decode_e4m3(qx) * np.repeat(sx.T.astype(np.float64), 128, 1)
    assert np.array_equal(y, deq_x)
    # E4M3 value times a power of two is a bf16 value: the bf16 output equals deq(Xq) exactly
    # (a sum that includes +0 products turns -0 into +0, hence the + 0.0)
    assert np.array_equal(bf16_round_from_f64(y), f32_to_bf16_bits((deq_x + 0.0).astype(np.float32)))
    # dgrad with W = I: dX = deq(dYq)
    assert np.array_equal(gemm_dgrad(qx, sx, qwt, sw), deq_x)


def test_permutation_and_scaled_identity_weights():
    xb = _rand((32, 256), 51)
    qx, sx = quant_act_1x128(xb, "cols")
    deq_x = decode_e4m3(qx) * np.repeat(sx.T.astype(np.float64), 128, 1)
    perm = np.random.default_rng(52).permutation(256)
    p = np.zeros((256, 256), np.float32)
    p[np.arange(256), perm] = 1.0  # W[n, perm[n]] = 1  ->  Y[:, n] = X[:, perm[n]]
    qw, _, sw = quant_w_128x128(_bits(p))
    assert np.array_equal(gemm_fprop(qx, sx, qw, sw), deq_x[:, perm])
    for t in (-20, -3, 5):
        qw2, _, sw2 = quant_w_128x128(_bits(np.eye(256, dtype=np.float32) * np.float32(2.0 ** t)))
        assert np.array_equal(gemm_fprop(qx, sx, qw2, sw2), deq_x * 2.0 ** t)


def test_one_hot_gradient_selects_rows_in_wgrad():
    xb = _rand((256, 128), 53)
    qxt, sx = quant_act_1x128(xb, "rows")
    deq_x = (decode_e4m3(qxt) * np.repeat(sx.T.astype(np.float64), 128, 1)).T  # [256 tokens, 128]
    pick = np.array([3, 200, 129, 64, 255])
    dy = np.zeros((256, 5), np.float32)
    dy[pick, np.arange(5)] = 1.0
    qdyt, sdy = quant_act_1x128(_bits(dy), "rows")
    dw = gemm_wgrad(qdyt, sdy, qxt, sx)
    assert np.array_equal(dw, deq_x[pick])


def test_worked_example_gemm():
    with open(GOLDEN) as f:
        ex = json.load(f)["gemm"]
    x = np.concatenate([np.full(128, 1.0), np.full(128, 0.25)])[None, :]
    w = np.zeros((128, 256))
    w[0, :] = 0.5
    w[1, :128] = -1.0
    w[1, 128:] = 2.0
    qx, sx = quant_act_1x128(_bits(x), "cols")
    qw, _, sw = quant_w_128x128(_bits(w))
    assert list(sx[:, 0]) == [2.0 ** -8, 2.0 ** -10] and list(sw[0]) == [2.0 ** -8, 2.0 ** -7]
    assert (qw[0, 0], qw[1, 0], qw[0, 200], qw[1, 200]) == (0x70, 0xF8, 0x68, 0x78)
    y = gemm_fprop(qx, sx, qw, sw)
    assert [y[0, 0], y[0, 1]] == [float(v) for v in ex["y"]]
    assert np.all(y[0, 2:] == 0.0)


def test_bf16_rounding_single_step():
    # values whose float32 rounding would double-round differently
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8 + 2.0 ** -40),
                  2.0 ** -130, 3 * 2.0 ** -134])
    got = bf16_round_from_f64(v)
    want = [0x3F81, 0x3F80, 0x3F82, 0xBF81, 0x0008, 0x0002]
    assert [int(g) for g in got] == want


def test_tolerance_report_flags_violations():
    ref = np.linspace(-1, 1, 1000)
    rep = gemm_tolerance_report(ref.astype(np.float32), ref)
    assert rep["violations"] == 0
    bad = ref.copy()
    bad[10] += 0.1
    assert gemm_tolerance_report(bad, ref)["violations"] == 1


@pytest.mark.parametrize("key", ["tiny_fprop", "attn_fprop", "mlp_gateup_fprop", "mlp_down_fprop_dgrad", "wgrad"])
def test_quantisation_error_sanity_bound(key):
    """||ref64 - A.B^T||_F / ||A.B^T||_F <= 0.05 on the configured distributions (rows truncated to 1024)."""
    t = generate(key)
    rows = 1024
    if key == "wgrad":
        dy, x = t["dY"][:rows], t["X"][:rows, :1024]
        qdyt, sdy = quant_act_1x128(dy, "rows")
        qxt, sx = quant_act_1x128(x, "rows")
        got = gemm_wgrad(qdyt, sdy, qxt, sx)
        ref = unquantized_reference(np.ascontiguousarray(dy.T), np.ascontiguousarray(x.T))
    else:
        x, w = t["X"][:rows], t["W"]
        qx, sx = quant_act_1x128(x, "cols")
        qw, qwt, sw = quant_w_128x128(w)
        got = gemm_fprop(qx, sx, qw, sw)
        ref = unquantized_reference(x, w)
        if key == "mlp_down_fprop_dgrad":
            dy = t["dY"][:rows]
            qdy, sdy = quant_act_1x128(dy, "cols")
            got2 = gemm_dgrad(qdy, sdy, qwt, sw)
            wt = np.ascontiguousarray(w.T)
            ref2 = unquantized_reference(dy, wt)
            assert np.linalg.norm(got2 - ref2) / np.linalg.norm(ref2) <= 0.05
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 0.05, rel


def test_workload_generator_recipe():
    t = generate("tiny_fprop")
    x = bf16_bits_to_f32(t["X"]).astype(np.float64)
    assert t["X"].shape == (256, 512) and t["W"].shape == (384, 512)
    # exactly round(0.005 * numel) entries were multiplied by 50: they are the ones far in the tail
    assert WORKLOADS["tiny_fprop"].spec("X").outlier_frac == 0.005
    assert np.count_nonzero(np.abs(x) > 8.0) <= 655 and np.count_nonzero(np.abs(x) > 8.0) > 500
    # asking for a subset yields the same bits
    assert np.array_equal(generate("tiny_fprop", only=["W"])["W"], t["W"])
    # same seed, same bits; the gate+up step shares X and W with the gate+up fprop workload
    a = generate("mlp_gateup_fprop", only=["X"])["X"]
    b = generate("mlp_gateup_layer_step", only=["X"])["X"]
    assert np.array_equal(a, b)


def test_unquantized_reference_brute_force_and_closed_forms():
    """The plain BF16 product A . B^T: small integers against an integer triple loop, identity and
    a hand-computed 2x2 example."""
    rng = np.random.default_rng(17)
    a = rng.integers(-8, 9, size=(5, 7)).astype(np.float32)
    b = rng.integers(-8, 9, size=(3, 7)).astype(np.float32)
    got = unquantized_reference(f32_to_bf16_bits(a), f32_to_bf16_bits(b))
    want = [[sum(int(a[i, k]) * int(b[j, k]) for k in range(7)) for j in range(3)] for i in range(5)]
    assert np.array_equal(got, np.array(want, dtype=np.float64))
    x = rng.standard_normal((4, 6)).astype(np.float32)
    xb = f32_to_bf16_bits(x)
    eye = f32_to_bf16_bits(np.eye(6, dtype=np.float32))
    assert np.array_equal(unquantized_reference(xb, eye), (xb.astype(np.uint32) << 16).view(np.float32))
    # [1.5, -2] . [[0.25, 4], [3, 0.5]]^T = [1.5*0.25 - 8, 4.5 - 1] = [-7.625, 3.5]
    two = unquantized_reference(f32_to_bf16_bits(np.array([[1.5, -2.0]], np.float32)),
                                f32_to_bf16_bits(np.array([[0.25, 4.0], [3.0, 0.5]], np.float32)))
    assert two.tolist() == [[-7.625, 3.5]]
