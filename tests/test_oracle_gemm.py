"""Pins for the oracle's block-scaled GEMM (CPU only).

Exact rational sums on tiny shapes, closed forms (identity, one-hot,
permutation and power-of-two-scaled weights), a hand-derived worked example,
the sanity bound on quantisation error against the unquantised product, and the
two parity checkers: the per-element bar and the accumulation contract.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (
    bf16_round_from_f64,
    contract_allowance,
    contract_report,
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


# The bar, per element: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), rms over every compared
# reference value. The bounds below are worked out by hand, with values chosen so that every
# quantity is exact in float64.

def test_tolerance_bound_is_inclusive_and_exact_at_its_edge():
    # ref = 1000 everywhere: rms = 1000, 1e-3 * rms = 1 exactly, 2^-7 * 1000 = 7.8125,
    # so the bound is 8.8125 for every element
    ref = np.full(4096, 1000.0)
    gpu = ref.copy()
    gpu[5] = 1000.0 + 8.8125   # on the bound, above
    gpu[6] = 1000.0 - 8.8125   # on the bound, below
    rep = gemm_tolerance_report(gpu, ref)
    assert rep["violations"] == 0
    assert rep["rms_ref"] == 1000.0 and rep["max_err_over_bound"] == 1.0
    gpu[7] = np.nextafter(1000.0 + 8.8125, np.inf)  # one float64 ulp past it
    gpu[8] = np.nextafter(1000.0 - 8.8125, -np.inf)
    assert gemm_tolerance_report(gpu, ref)["violations"] == 2


def test_tolerance_bound_separates_adjacent_bf16_values():
    # ref = 896 everywhere (a bf16 value; bf16 spacing is 4 in [512, 1024)):
    # bound = 2^-7 * 896 + 1e-3 * 896 = 7 + 0.896 = 7.896, so the bf16 neighbours 900 and 892
    # (error 4) pass while 904 and 888 (error 8), one bf16 ulp further, fail
    ref = np.full(64, 896.0)
    for ok_val, bad_val in ((900.0, 904.0), (892.0, 888.0)):
        gpu = ref.copy()
        gpu[3] = ok_val
        assert gemm_tolerance_report(gpu, ref)["violations"] == 0
        gpu[3] = bad_val
        assert gemm_tolerance_report(gpu, ref)["violations"] == 1


def test_tolerance_relative_term_is_two_to_minus_seven():
    # one large reference value among zeros: ref = [256, 0 x 65535], rms = 256 / 256 = 1,
    # bound at element 0 = 2 + 0.001; an error of 3 is outside 2^-7 * 256 + 1e-3 but would be
    # inside 2^-6 * 256 + 1e-3 = 4.001, and an error of 2 is inside
    ref = np.zeros(65536)
    ref[0] = 256.0
    gpu = ref.copy()
    gpu[0] = 258.0
    assert gemm_tolerance_report(gpu, ref)["violations"] == 0
    gpu[0] = 259.0
    rep = gemm_tolerance_report(gpu, ref)
    assert rep["violations"] == 1 and rep["rms_ref"] == 1.0
    assert abs(rep["max_err_over_bound"] - 3.0 / 2.001) < 1e-12


def test_tolerance_absolute_term_uses_the_reference_rms():
    # ref = [1, 0 x 999]: rms(ref) = sqrt(1/1000) = 0.0316..., so the bound at a zero reference
    # is 3.16e-5. gpu carries a gross error of 100 at element 1 (a violation whichever rms is
    # used) and an error of 1e-3 at element 2: outside 1e-3 * rms(ref) = 3.2e-5, but inside
    # 1e-3 * rms(gpu) = 1e-3 * sqrt((1 + 100^2 + 1e-6) / 1000) = 3.2e-3. Taking the rms over the
    # GPU values would hide the second violation.
    ref = np.zeros(1000)
    ref[0] = 1.0
    gpu = ref.copy()
    gpu[1] = 100.0
    gpu[2] = 1e-3
    rep = gemm_tolerance_report(gpu, ref)
    assert rep["violations"] == 2
    assert abs(rep["rms_ref"] - np.sqrt(1e-3)) < 1e-15
    # an all-zero reference has rms 0: only exact zeros pass
    z = np.zeros(8)
    assert gemm_tolerance_report(z, z)["violations"] == 0
    assert gemm_tolerance_report(np.full(8, 2.0 ** -149), z)["violations"] == 8


@pytest.mark.parametrize("key", ["tiny_fprop", "attn_fprop", "mlp_gateup_fprop", "mlp_down_fprop_dgrad", "wgrad"])
def test_quantisation_error_sanity_bound(key):
    """||ref64 - A.B^T||_F / ||A.B^T||_F <= 0.05 on every configuration at its full size (the
    oracle's block-scaled product against the float64 product of the unquantised bf16 inputs)."""
    t = generate(key)

    def rel(got, ref):
        return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))

    if key == "wgrad":
        dy, x = t["dY"], t["X"]
        qdyt, sdy = quant_act_1x128(dy, "rows")
        qxt, sx = quant_act_1x128(x, "rows")
        r = rel(gemm_wgrad(qdyt, sdy, qxt, sx), unquantized_reference(np.ascontiguousarray(dy.T), np.ascontiguousarray(x.T)))
        assert r <= 0.05, r
        return
    x, w = t["X"], t["W"]
    qx, sx = quant_act_1x128(x, "cols")
    qw, qwt, sw = quant_w_128x128(w)
    r = rel(gemm_fprop(qx, sx, qw, sw), unquantized_reference(x, w))
    assert r <= 0.05, r
    if key == "mlp_down_fprop_dgrad":
        dy = t["dY"]
        qdy, sdy = quant_act_1x128(dy, "cols")
        r2 = rel(gemm_dgrad(qdy, sdy, qwt, sw), unquantized_reference(dy, np.ascontiguousarray(w.T)))
        assert r2 <= 0.05, r2


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


# ---- accumulation contract (oracle.contract_allowance) ----
# The allowance states what FP32 accumulation on a matrix unit with an 8-product fixed-point
# window delivers: per group, products truncated toward zero to multiples of 2^(E-13) below the
# group's largest product 2^E <= max|p| < 2^(E+1). The pins below check it against a scalar loop
# and against a plain model of such an accumulator, including the model's worst case.

def _window_model(a_row, b_row):
    """Dot product as the windowed accumulator forms it: exact products, per group of 8 each
    truncated toward zero to a multiple of 2^(E-13), group sums added in float32, then RNE to bf16
    (as float64)."""
    acc = np.float32(0.0)
    for g in range(0, len(a_row), 8):
        p = [Fraction(float(a_row[k])) * Fraction(float(b_row[k])) for k in range(g, g + 8)]
        big = max(abs(x) for x in p)
        if big == 0:
            continue
        e = big.numerator.bit_length() - big.denominator.bit_length()
        if Fraction(2) ** e > big:
            e -= 1
        lsb = Fraction(2) ** (e - 13)
        s = sum((abs(x) // lsb) * lsb * (1 if x >= 0 else -1) for x in p)
        acc = np.float32(acc + np.float32(float(s)))
    bits = int(bf16_round_from_f64(np.array([float(acc)]))[0])
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def test_contract_allowance_matches_a_scalar_loop():
    rng = np.random.default_rng(41)
    a = rng.standard_normal((3, 32)) * np.where(rng.random((3, 32)) < 0.1, 50.0, 1.0)
    b = rng.standard_normal((4, 32))
    ref = a @ b.T
    got = contract_allowance(a, b, ref)
    for i in range(3):
        for j in range(4):
            gmax = sum(max(abs(a[i, k] * b[j, k]) for k in range(g, g + 8)) for g in range(0, 32, 8))
            asum = sum(abs(a[i, k] * b[j, k]) for k in range(32))
            want = 2.0 ** -8 * abs(ref[i, j]) + (1 + 2.0 ** -8) * (7 * 2.0 ** -13 * gmax + 8 * 2.0 ** -24 * asum)
            assert abs(got[i, j] - want) <= 1e-15 * want


def test_contract_allowance_closed_form():
    # one row: 448 at k = 0 and seven products of 2^-6 in the same group, zeros elsewhere (K = 128);
    # sum_g max = 448, sum |p| = 448 + 7 * 2^-6, ref = 448 + 7 * 2^-6
    a = np.zeros((1, 128))
    a[0, 0] = 448.0
    a[0, 1:8] = 2.0 ** -6
    b = np.ones((1, 128))
    ref = a @ b.T
    want = 2.0 ** -8 * ref[0, 0] + (1 + 2.0 ** -8) * (7 * 2.0 ** -13 * 448 + 32 * 2.0 ** -24 * ref[0, 0])
    assert contract_allowance(a, b, ref)[0, 0] == want
    # the window model drops all seven small products (each below 2^(8-13) = 2^-5): error 7 * 2^-6,
    # inside the allowance
    model = _window_model(a[0], b[0])
    assert model == 448.0 and abs(model - ref[0, 0]) <= want


def test_contract_allowance_holds_for_the_window_model_and_is_nearly_tight():
    # random operands with outliers in both, every element of the model inside the allowance
    rng = np.random.default_rng(43)
    vals = np.array([decode_e4m3(np.array([c], np.uint8))[0] for c in range(256) if (c & 0x7F) != 0x7F])
    a = rng.choice(vals, size=(6, 64)) * np.where(rng.random((6, 64)) < 0.05, 16.0, 1.0)
    b = rng.choice(vals, size=(5, 64))
    ref = a @ b.T
    allow = contract_allowance(a, b, ref)
    model = np.array([[_window_model(a[i], b[j]) for j in range(5)] for i in range(6)])
    assert contract_report(model, ref, allow)["violations"] == 0
    # worst case of one group, no bf16 rounding: max product exactly 2^8, seven products just
    # below the window's quantum 2^-5 (largest E4M3 value under 2^-5 is 0.029296875 = 15 * 2^-9)
    a = np.zeros((1, 8))
    a[0, 0] = 256.0
    a[0, 1:] = 15 * 2.0 ** -9
    b = np.ones((1, 8))
    ref = a @ b.T
    err = abs(_window_model(a[0], b[0]) - ref[0, 0])   # every small product is dropped
    assert err == 7 * 15 * 2.0 ** -9
    window_part = contract_allowance(a, b, ref)[0, 0] - 2.0 ** -8 * ref[0, 0]
    assert err <= window_part and err / window_part > 0.9  # 6/7 of the allowance or more would fail a looser 2^-14


def test_contract_report_counts_elements_outside_the_allowance():
    ref = np.array([1.0, 2.0, 3.0, 4.0])
    allow = np.array([0.5, 0.5, 0.5, 0.0])
    gpu = np.array([1.5, 2.5000001, 2.5, 4.0])
    rep = contract_report(gpu, ref, allow)
    assert rep["violations"] == 1 and rep["n"] == 4
    assert abs(rep["max_err_over_allowance"] - 0.5000001 / 0.5) < 1e-12
