"""GPU block-scaled GEMM vs the CPU oracle (runs on an MI355X).

Two bounds, both stated in include/pf8.h (ref = the unrounded float64 oracle value on the same
codes; the GPU quantisers' codes are checked bit-exact against the oracle's first):
- the per-element bar |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), for operands distributed like
  the workloads (outliers in the activations only);
- the accumulation contract oracle.contract_allowance, which holds for any operands, for tests
  that put outliers (or arbitrary codes) in both operands.
At the configured full sizes the oracle computes a seeded sample of output rows (spread over
every row tile) against the complete columns.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_pf8_amd as pf8
import oracle
from workloads import WORKLOADS, f32_to_bf16_bits, generate
from tests.gpu_helpers import DEV, bf16_bits, bf16_f64, f32, to_dev_bf16, to_dev_f32, to_dev_u8, u8

pytestmark = pytest.mark.gpu

VARIANTS = [pf8.PF8_GEMM_MX_SCALED, pf8.PF8_GEMM_PROMOTE]
VNAME = {pf8.PF8_GEMM_MX_SCALED: "mx", pf8.PF8_GEMM_PROMOTE: "promote"}


def _report(gpu_d, ref, what):
    rep = oracle.gemm_tolerance_report(gpu_d, ref)
    assert rep["violations"] == 0, f"{what}: {rep}"
    # diagnostic, not the bar: most outputs round to the same bf16 as the float64 value
    if rep["n"] >= 1000:
        assert rep["frac_bit_equal_bf16"] > 0.95, f"{what}: {rep}"
    return rep


def _contract(gpu_d, ref, a_deq, b_deq, what):
    """The accumulation contract for any operands: a_deq [rows, K] / b_deq [n, K] dequantised."""
    rep = oracle.contract_report(gpu_d, ref, oracle.contract_allowance(a_deq, b_deq, ref))
    assert rep["violations"] == 0, f"{what}: {rep}"
    return rep


def _sample_rows(m, n_sample, seed):
    if m <= n_sample:
        return np.arange(m)
    return np.sort(np.random.default_rng(seed).choice(m, n_sample, replace=False))


def _quant_all_gpu(x_bits=None, w_bits=None, dy_bits=None):
    """GPU quantisers on whichever inputs are given (each mode only where its shape allows it)."""
    out = {}
    for name, bits in (("x", x_bits), ("dy", dy_bits)):
        if bits is None:
            continue
        t = to_dev_bf16(bits)
        if bits.shape[1] % 128 == 0:
            out["q" + name], out["s" + name] = pf8.quant_act_1x128(t, "cols")
        if bits.shape[0] % 128 == 0 and bits.shape[1] % 8 == 0:
            out["q" + name + "t"], out["s" + name + "t"] = pf8.quant_act_1x128(t, "rows")
    if w_bits is not None:
        out["qw"], out["qwt"], out["sw"] = pf8.quant_w_128x128(to_dev_bf16(w_bits))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("key", ["tiny_fprop", "attn_fprop", "mlp_gateup_fprop", "mlp_down_fprop_dgrad"])
def test_fprop_workloads(key, variant):
    t = generate(key, only=["X", "W"])
    g = _quant_all_gpu(x_bits=t["X"], w_bits=t["W"])
    qx, sx = oracle.quant_act_1x128(t["X"], "cols")
    qw, qwt, sw = oracle.quant_w_128x128(t["W"])
    assert np.array_equal(u8(g["qx"]), qx) and np.array_equal(u8(g["qw"]), qw)
    y = pf8.fprop(g["qx"], g["sx"], g["qw"], g["sw"], variant=variant)
    torch.cuda.synchronize()
    rows = _sample_rows(qx.shape[0], 384, 11)
    ref = oracle.gemm_fprop(qx[rows], sx[:, rows], qw, sw)
    _report(bf16_f64(y)[rows], ref, f"{key} fprop")


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_dgrad_workload(variant):
    t = generate("mlp_down_fprop_dgrad", only=["W", "dY"])
    g = _quant_all_gpu(w_bits=t["W"], dy_bits=t["dY"])
    qdy, sdy = oracle.quant_act_1x128(t["dY"], "cols")
    qw, qwt, sw = oracle.quant_w_128x128(t["W"])
    assert np.array_equal(u8(g["qdy"]), qdy) and np.array_equal(u8(g["qwt"]), qwt)
    dx = pf8.dgrad(g["qdy"], g["sdy"], g["qwt"], g["sw"], variant=variant)
    torch.cuda.synchronize()
    rows = _sample_rows(qdy.shape[0], 384, 12)
    ref = oracle.gemm_dgrad(qdy[rows], sdy[:, rows], qwt, sw)
    _report(bf16_f64(dx)[rows], ref, "dgrad")


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_wgrad_workload(variant):
    t = generate("wgrad")
    g = _quant_all_gpu(x_bits=t["X"], dy_bits=t["dY"])
    qdyt, sdy = oracle.quant_act_1x128(t["dY"], "rows")
    qxt, sx = oracle.quant_act_1x128(t["X"], "rows")
    assert np.array_equal(u8(g["qdyt"]), qdyt) and np.array_equal(u8(g["qxt"]), qxt)
    dw = pf8.wgrad(g["qdyt"], g["sdyt"], g["qxt"], g["sxt"], variant=variant)
    torch.cuda.synchronize()
    rows = _sample_rows(qdyt.shape[0], 256, 13)
    ref = oracle.gemm_wgrad(qdyt[rows], sdy[:, rows], qxt, sx)
    _report(bf16_f64(dw)[rows], ref, "wgrad")


def _rand_bits(shape, seed, sigma=1.0, outliers=True):
    """N(0, sigma) bf16; with `outliers`, 0.5 % of the entries x50 (the activation model of the
    workloads; weights and gradients are drawn without)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    if outliers:
        x.reshape(-1)[rng.choice(x.size, max(1, x.size // 200), replace=False)] *= 50
    return f32_to_bf16_bits(x)


SHAPES = [(1, 1, 128), (1, 130, 256), (3, 5, 128), (300, 200, 384), (257, 129, 256), (513, 777, 640),
          (256, 384, 512), (640, 448, 256), (129, 1000, 128),
          # ragged in both M and N, sized so that the launcher's tile choice (fewest rounds of one
          # tile per CU, weighted by tile area) lands on each macro-tile: 256x128, 256x192,
          # 192x256 and 256x256 (the shapes above all take 128x128)
          (644, 5407, 384), (1421, 5407, 256), (2050, 5407, 384), (2309, 4874, 640)]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_ragged_shapes_all_layouts(m, n, k, variant):
    """Ragged M and N (any value) with K a multiple of 128: all three layouts, full outputs."""
    # fprop: A = X [m, k] row codes, B = W [n', k] tile codes with n' padded to 128 rows
    xb = _rand_bits((m, k), m * 7 + n)
    n_pad = (n + 127) // 128 * 128
    wb = _rand_bits((n_pad, k), n * 3 + k, 0.02, outliers=False)
    qx, sx = oracle.quant_act_1x128(xb, "cols")
    qw, qwt, sw = oracle.quant_w_128x128(wb)
    d = pf8.fprop(to_dev_u8(qx), to_dev_f32(sx), to_dev_u8(qw[:n]), to_dev_f32(sw), variant=variant)
    torch.cuda.synchronize()
    _report(bf16_f64(d), oracle.gemm_fprop(qx, sx, qw[:n], sw), f"fprop {m}x{n}x{k}")
    # dgrad: A = dY [m, k'] along its columns; B = W^T codes [n, k'] (first n rows), W tile grid [k'/128, *]
    wb2 = _rand_bits((k, n_pad), k + n, 0.01, outliers=False)  # W [Nw = k, Kw = n_pad]
    q2, qt2, sw2 = oracle.quant_w_128x128(wb2)
    dyb = _rand_bits((m, k), m + 5, 1e-3, outliers=False)
    qdy, sdy = oracle.quant_act_1x128(dyb, "cols")
    d = pf8.dgrad(to_dev_u8(qdy), to_dev_f32(sdy), to_dev_u8(qt2[:n]), to_dev_f32(sw2), variant=variant)
    torch.cuda.synchronize()
    _report(bf16_f64(d), oracle.gemm_dgrad(qdy, sdy, qt2[:n], sw2), f"dgrad {m}x{n}x{k}")
    # wgrad: A = dY^T codes [m, k] grouped along k (tokens), B = X^T codes [n, k]
    dyt = _rand_bits((k, m + (-m % 8)), m + 11, 1e-3, outliers=False)
    xt = _rand_bits((k, n + (-n % 8)), n + 13)
    qa, sa = oracle.quant_act_1x128(dyt, "rows")
    qb, sb = oracle.quant_act_1x128(xt, "rows")
    d = pf8.wgrad(to_dev_u8(qa[:m]), to_dev_f32(sa), to_dev_u8(qb[:n]), to_dev_f32(sb), variant=variant)
    torch.cuda.synchronize()
    _report(bf16_f64(d), oracle.gemm_wgrad(qa[:m], sa[:, :m], qb[:n], sb[:, :n]), f"wgrad {m}x{n}x{k}")


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_ragged_shapes_outliers_in_both_operands(m, n, k, variant):
    """The ragged shapes above with 0.5 % x50 outliers in W and dY as well (every operand
    heavy-tailed): all three layouts inside the accumulation contract, on every output row up
    to 256 rows and on 128 sampled rows (first and last included) beyond."""
    rows = np.arange(m) if m <= 256 else np.unique(np.concatenate([[0, m - 1], _sample_rows(m, 128, m + n)]))
    n_pad = (n + 127) // 128 * 128
    qx, sx = oracle.quant_act_1x128(_rand_bits((m, k), m * 7 + n), "cols")
    qw, _, sw = oracle.quant_w_128x128(_rand_bits((n_pad, k), n * 3 + k, 0.02))
    d = pf8.fprop(to_dev_u8(qx), to_dev_f32(sx), to_dev_u8(qw[:n]), to_dev_f32(sw), variant=variant)
    torch.cuda.synchronize()
    _contract(bf16_f64(d)[rows], oracle.gemm_fprop(qx[rows], sx[:, rows], qw[:n], sw),
              oracle.dequant_act_groups(qx[rows], sx[:, rows]), oracle.dequant_w_tiles(qw[:n], sw),
              f"fprop {m}x{n}x{k}")
    _, qt2, sw2 = oracle.quant_w_128x128(_rand_bits((k, n_pad), k + n, 0.01))
    qdy, sdy = oracle.quant_act_1x128(_rand_bits((m, k), m + 5, 1e-3), "cols")
    d = pf8.dgrad(to_dev_u8(qdy), to_dev_f32(sdy), to_dev_u8(qt2[:n]), to_dev_f32(sw2), variant=variant)
    torch.cuda.synchronize()
    _contract(bf16_f64(d)[rows], oracle.gemm_dgrad(qdy[rows], sdy[:, rows], qt2[:n], sw2),
              oracle.dequant_act_groups(qdy[rows], sdy[:, rows]), oracle.dequant_w_tiles(qt2[:n], sw2.T),
              f"dgrad {m}x{n}x{k}")
    qa, sa = oracle.quant_act_1x128(_rand_bits((k, m + (-m % 8)), m + 11, 1e-3), "rows")
    qb, sb = oracle.quant_act_1x128(_rand_bits((k, n + (-n % 8)), n + 13), "rows")
    d = pf8.wgrad(to_dev_u8(qa[:m]), to_dev_f32(sa), to_dev_u8(qb[:n]), to_dev_f32(sb), variant=variant)
    torch.cuda.synchronize()
    _contract(bf16_f64(d)[rows], oracle.gemm_wgrad(qa[rows], sa[:, rows], qb[:n], sb[:, :n]),
              oracle.dequant_act_groups(qa[rows], sa[:, rows]), oracle.dequant_act_groups(qb[:n], sb[:, :n]),
              f"wgrad {m}x{n}x{k}")


# gfx950's FP8 MFMA (scaled and unscaled) adds the products of each aligned group of 8
# consecutive K values in a fixed-point window: every product is truncated toward zero to a
# multiple of 2^(E-13), E = floor(log2) of the group's largest product magnitude, and the group
# sums accumulate in FP32. With outliers in one operand only (the workloads: activations) results
# stay inside 2^-7 |ref| + 1e-3 rms(ref); with outliers in both, a group holding an outlier
# product can lose its other products' low bits. include/pf8.h states the resulting accumulation
# contract (oracle.contract_allowance); the tests below pin the window and check the contract.

def _chunk_gemm(variant, a_codes_at, k=128, b_code=0x38):
    """One output element: A row of zeros with the given (position, code) entries, B all b_code,
    unit scales."""
    a = np.zeros((1, k), np.uint8)
    for pos, code in a_codes_at:
        a[0, pos] = code
    b = np.full((1, k), b_code, np.uint8)
    d = pf8.fprop(to_dev_u8(a), to_dev_f32(np.ones((k // 128, 1), np.float32)), to_dev_u8(b),
                  to_dev_f32(np.ones((1, k // 128), np.float32)), variant=variant)
    torch.cuda.synchronize()
    return float(bf16_f64(d)[0, 0])


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_mfma_chunk_precision(variant):
    big, nbig = 0x7E, 0xFE  # +-448 = 1.75 * 2^8: the window's quantum beside it is 2^-5
    # small terms in a group of their own, and sums whose terms all fit the window, are exact
    assert _chunk_gemm(variant, [(0, 0x01)]) == 2.0 ** -9  # E4M3 subnormals are honoured
    assert _chunk_gemm(variant, [(0, big), (1, 0x38), (2, nbig)]) == 1.0
    assert _chunk_gemm(variant, [(0, big), (1, 0x20), (127, nbig)]) == 0.125
    assert _chunk_gemm(variant, [(0, big), (8, 0x08), (16, nbig)]) == 2.0 ** -6  # k = 8 starts a new group
    assert _chunk_gemm(variant, [(0, big), (130, 0x01), (300, nbig)], k=384) == 2.0 ** -9
    # inside the group of 448 (k = 0..7), products are truncated toward zero to multiples of 2^-5
    assert _chunk_gemm(variant, [(0, big), (7, 0x08), (40, nbig)]) == 0.0            # 2^-6 -> 0
    assert _chunk_gemm(variant, [(0, big), (1, 0x23), (40, nbig)]) == 0.15625        # 0.171875 -> 5 * 2^-5
    assert _chunk_gemm(variant, [(0, big), (1, 0xA3), (40, nbig)]) == -0.15625       # toward zero, not down
    # each product on its own: 2 x 0.05859375 -> 2 x 2^-5 (the truncated sum would be 3 x 2^-5)
    assert _chunk_gemm(variant, [(0, big), (1, 0x17), (2, 0x17), (40, nbig)]) == 0.0625
    # the window follows the largest magnitude even when it cancels inside the group
    assert _chunk_gemm(variant, [(0, big), (1, nbig), (2, 0x08)]) == 0.0
    # and scales with it: beside 1.0 (E = 0) the quantum is 2^-13, so 2^-9 survives
    assert _chunk_gemm(variant, [(0, 0x38), (1, 0x01), (40, 0xB8)]) == 2.0 ** -9


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("m,n,k", [(2309, 4874, 640), (1024, 1024, 4096)])
def test_heavy_tailed_operands_within_chunk_bound(m, n, k, variant):
    """dgrad with 0.5 % x50 outliers in both dY and W (harsher than the workloads): sampled rows,
    the first and last included, inside the accumulation contract."""
    n_pad = (n + 127) // 128 * 128
    wb = _rand_bits((k, n_pad), k + n, 0.01)
    qw, qwt, sw = oracle.quant_w_128x128(wb)
    dyb = _rand_bits((m, k), m + 5, 1e-3)
    qdy, sdy = oracle.quant_act_1x128(dyb, "cols")
    d = pf8.dgrad(to_dev_u8(qdy), to_dev_f32(sdy), to_dev_u8(qwt[:n]), to_dev_f32(sw), variant=variant)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], _sample_rows(m, 128, m + k)]))
    ref = oracle.gemm_dgrad(qdy[rows], sdy[:, rows], qwt[:n], sw)
    _contract(bf16_f64(d)[rows], ref, oracle.dequant_act_groups(qdy[rows], sdy[:, rows]),
              oracle.dequant_w_tiles(qwt[:n], sw.T), f"dgrad {m}x{n}x{k}")


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_identity_weight_reproduces_dequantised_input(variant):
    xb = _rand_bits((512, 512), 21)
    qx, sx = oracle.quant_act_1x128(xb, "cols")
    eye = f32_to_bf16_bits(np.eye(512, dtype=np.float32))
    g = _quant_all_gpu(w_bits=eye)
    y = pf8.fprop(to_dev_u8(qx), to_dev_f32(sx), g["qw"], g["sw"], variant=variant)
    dx = pf8.dgrad(to_dev_u8(qx), to_dev_f32(sx), g["qwt"], g["sw"], variant=variant)
    torch.cuda.synchronize()
    deq = oracle.decode_e4m3(qx) * np.repeat(sx.T.astype(np.float64), 128, 1) + 0.0
    want = f32_to_bf16_bits(deq.astype(np.float32))
    assert np.array_equal(bf16_bits(y), want)
    assert np.array_equal(bf16_bits(dx), want)


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_one_hot_gradient_selects_rows_in_wgrad(variant):
    xb = _rand_bits((256, 384), 22)
    pick = np.array([0, 255, 17, 128, 129, 64, 200, 3])
    dy = np.zeros((256, 8), np.float32)
    dy[pick, np.arange(8)] = 1.0
    g = _quant_all_gpu(x_bits=xb, dy_bits=f32_to_bf16_bits(dy))
    dw = pf8.wgrad(g["qdyt"], g["sdyt"], g["qxt"], g["sxt"], variant=variant)
    torch.cuda.synchronize()
    qxt, sxt = oracle.quant_act_1x128(xb, "rows")
    deq_x = (oracle.decode_e4m3(qxt) * np.repeat(sxt.T.astype(np.float64), 128, 1)).T + 0.0
    assert np.array_equal(bf16_bits(dw), f32_to_bf16_bits(deq_x[pick].astype(np.float32)))


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_small_integer_block_is_exact(variant):
    """Single and multi-block GEMMs whose FP32 sums are exact: the GPU must equal the exact value."""
    rng = np.random.default_rng(5)
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0xC8], np.uint8)  # 0, +-1, +-2, +-3, +-4
    # products are multiples of 2^-4 below 2^8 and |sums| stay below 2^18: every partial sum is an fp32 value
    for m, n, k in [(64, 64, 128), (256, 256, 512), (300, 260, 1024)]:
        qa = rng.choice(ints, size=(m, k))
        qb = rng.choice(ints, size=(n, k))
        sa = np.ldexp(1.0, rng.integers(-2, 3, size=(k // 128, m))).astype(np.float32)
        sb = np.ldexp(1.0, rng.integers(-2, 3, size=((n + 127) // 128, k // 128))).astype(np.float32)
        d = pf8.fprop(to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb), variant=variant)
        torch.cuda.synchronize()
        ref = oracle.gemm_fprop(qa, sa, qb, sb)  # exact: small integers times powers of two
        want = oracle.bf16_round_from_f64(ref)
        assert np.array_equal(bf16_bits(d), want), f"{m}x{n}x{k}"


def test_variants_agree_and_repeat_bitwise():
    t = generate("tiny_fprop")
    g = _quant_all_gpu(x_bits=t["X"], w_bits=t["W"])
    outs = [pf8.fprop(g["qx"], g["sx"], g["qw"], g["sw"], variant=pf8.PF8_GEMM_MX_SCALED) for _ in range(3)]
    auto = pf8.fprop(g["qx"], g["sx"], g["qw"], g["sw"])
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert torch.equal(auto, outs[0])


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: VNAME[v])
def test_padded_output_and_strided_operands(variant):
    """lda > k, ld_as > m and ldd > n: bytes outside D's [m, n] window stay untouched."""
    m, n, k = 200, 300, 256
    xb = _rand_bits((m, k), 31)
    wb = _rand_bits((384, k), 32, 0.02, outliers=False)
    qx, sx = oracle.quant_act_1x128(xb, "cols")
    qw, _, sw = oracle.quant_w_128x128(wb)
    a = np.zeros((m, 272), np.uint8)
    a[:, :k] = qx
    sa = np.zeros((2, 208), np.float32)
    sa[:, :m] = sx
    a_d, sa_d = to_dev_u8(a), to_dev_f32(sa)
    b_d, sb_d = to_dev_u8(qw), to_dev_f32(sw)
    canary = 0x7FC1  # a bf16 NaN pattern nothing writes
    d = torch.full((m + 3, 312), canary, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pf8._lib.check(pf8.pf8_block_gemm_variant(variant, pf8.PF8_FPROP, m, n, k, a_d.data_ptr(), 272, sa_d.data_ptr(),
                                              208, b_d.data_ptr(), k, sb_d.data_ptr(), sw.shape[1], 1, d.data_ptr(),
                                              312, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    bits = bf16_bits(d)
    assert np.all(bits[:m, n:] == canary) and np.all(bits[m:, :] == canary)
    got = (bits[:m, :n].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _report(got, oracle.gemm_fprop(qx, sx, qw[:n], sw), "strided")


@pytest.mark.parametrize("fused", [True, False], ids=["dual_quant", "single_quant"])
def test_linear_step_matches_oracle(fused):
    """The whole layer pass used by the benchmark on the tiny shape, with the fused quantisers (5
    launches) and with one quantiser pass per orientation (8 launches)."""
    t = generate("tiny_fprop")
    dyb = _rand_bits((256, 384), 41, 1e-3, outliers=False)
    step = pf8.LinearStep(to_dev_bf16(t["X"]), to_dev_bf16(t["W"]), to_dev_bf16(dyb), fused=fused)
    assert len(step.launches()) == (5 if fused else 8)
    step.run()
    torch.cuda.synchronize()
    qx, sx = oracle.quant_act_1x128(t["X"], "cols")
    qw, qwt, sw = oracle.quant_w_128x128(t["W"])
    qdy, sdy = oracle.quant_act_1x128(dyb, "cols")
    qdyt, sdyt = oracle.quant_act_1x128(dyb, "rows")
    qxt, sxt = oracle.quant_act_1x128(t["X"], "rows")
    _report(bf16_f64(step.y), oracle.gemm_fprop(qx, sx, qw, sw), "step fprop")
    _report(bf16_f64(step.dx), oracle.gemm_dgrad(qdy, sdy, qwt, sw), "step dgrad")
    _report(bf16_f64(step.dw), oracle.gemm_wgrad(qdyt, sdyt, qxt, sxt), "step wgrad")


@pytest.mark.parametrize("fused", [True, False], ids=["dual_quant", "single_quant"])
def test_linear_step_reusing_weight_codes(fused):
    """A later micro-batch's step (W's codes from an earlier run, one launch fewer) gives the full
    step's results bit for bit."""
    t = generate("tiny_fprop")
    dyb = _rand_bits((256, 384), 47, 1e-3, outliers=False)
    step = pf8.LinearStep(to_dev_bf16(t["X"]), to_dev_bf16(t["W"]), to_dev_bf16(dyb), fused=fused)
    assert len(step.launches(weight_codes=False)) == len(step.launches()) - (0 if fused else 1)
    step.run()
    torch.cuda.synchronize()
    outs = lambda: [o.clone() for o in (step.y, step.dx, step.dw, step.qx, step.qxt, step.sx, step.sxt)]  # noqa: E731
    want = outs()
    for o in (step.y, step.dx, step.dw):
        o.fill_(float("nan"))
    for o in (step.qx, step.qxt, step.sx, step.sxt):
        o.fill_(0)
    step.run(weight_codes=False)
    torch.cuda.synchronize()
    for got, ref in zip(outs(), want):
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))


def test_linear_step_on_a_side_stream_and_in_a_graph():
    """The library enqueues on the caller's stream and allocates nothing, so the step runs on a
    side stream and replays from a captured HIP graph. Every replay (with eager work in between
    that overwrites the results) equals the eager default-stream run bit for bit."""
    t = generate("tiny_fprop")
    dyb = _rand_bits((256, 384), 43, 1e-3, outliers=False)
    step = pf8.LinearStep(to_dev_bf16(t["X"]), to_dev_bf16(t["W"]), to_dev_bf16(dyb))
    outs = lambda: [o.clone() for o in (step.y, step.dx, step.dw, step.qx, step.qdyt, step.sxt)]  # noqa: E731
    step.run()
    torch.cuda.synchronize()
    want = outs()
    side = torch.cuda.Stream()
    for o in (step.y, step.dx, step.dw):
        o.fill_(float("nan"))
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    side.synchronize()
    for got, ref in zip(outs(), want):
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
    graph = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()  # warm-up on the capturing side stream, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step.run()
    for rep in range(3):
        for o in (step.y, step.dx, step.dw):
            o.fill_(float("nan"))
        step.qx.fill_(0)
        step.sxt.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs(), want):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"replay {rep}"


def test_linear_steps_from_concurrent_host_threads():
    """The ABI keeps no state, so host threads may enqueue at once: four threads, each with its own
    layer step on its own stream, run 10 steps each; every result equals the step's lone run."""
    import threading
    t = generate("tiny_fprop")
    steps = []
    for i in range(4):
        dyb = _rand_bits((256, 384), 50 + i, 1e-3, outliers=False)
        x = to_dev_bf16(t["X"]) * (1.0 + 0.25 * i)
        steps.append(pf8.LinearStep(x, to_dev_bf16(t["W"]), to_dev_bf16(dyb)))
    outs = lambda st: [o.clone() for o in (st.y, st.dx, st.dw, st.qxt, st.sdyt)]  # noqa: E731
    want = []
    for st in steps:
        st.run()
        torch.cuda.synchronize()
        want.append(outs(st))
        for o in (st.y, st.dx, st.dw):
            o.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in steps]
    errors = []

    def worker(st, stream):
        try:
            with torch.cuda.stream(stream):
                for _ in range(10):
                    st.run()
        except Exception as e:  # reported below, on the test's thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(st, sm)) for st, sm in zip(steps, streams)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors and not any(th.is_alive() for th in threads), errors
    for i, st in enumerate(steps):
        for got, ref in zip(outs(st), want[i]):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"step {i}"


def test_layer_step_workload_sampled():
    """The benchmark's gate+up layer pass at full size: sampled codes and outputs against the oracle.

    Row-mode groups live in one row and col-mode groups in one column, so the oracle quantises
    just the sampled rows / columns of dY."""
    wl = WORKLOADS["mlp_gateup_layer_step"]
    t = generate(wl)
    step = pf8.LinearStep(to_dev_bf16(t["X"]), to_dev_bf16(t["W"]), to_dev_bf16(t["dY"]))
    step.run()
    torch.cuda.synchronize()
    rows = _sample_rows(8192, 128, 51)
    qx, sx = oracle.quant_act_1x128(t["X"], "cols")
    qw, qwt, sw = oracle.quant_w_128x128(t["W"])
    assert np.array_equal(u8(step.qx), qx) and np.array_equal(u8(step.qw), qw) and np.array_equal(u8(step.qwt), qwt)
    _report(bf16_f64(step.y)[rows], oracle.gemm_fprop(qx[rows], sx[:, rows], qw, sw), "layer fprop")
    qdy, sdy = oracle.quant_act_1x128(np.ascontiguousarray(t["dY"][rows]), "cols")
    assert np.array_equal(u8(step.qdy)[rows], qdy) and np.array_equal(f32(step.sdy)[:, rows], sdy)
    _report(bf16_f64(step.dx)[rows], oracle.gemm_dgrad(qdy, sdy, qwt, sw), "layer dgrad")
    cols = _sample_rows(12288, 128, 52)
    qdyt, sdyt = oracle.quant_act_1x128(np.ascontiguousarray(t["dY"][:, cols]), "rows")
    qxt, sxt = oracle.quant_act_1x128(t["X"], "rows")
    assert np.array_equal(u8(step.qdyt)[cols], qdyt) and np.array_equal(u8(step.qxt), qxt)
    _report(bf16_f64(step.dw)[cols], oracle.gemm_wgrad(qdyt, sdyt, qxt, sxt), "layer wgrad")


# ---- FP32 results (pf8_block_gemm_f32): same products, no BF16 rounding, optional accumulate ----

def _operands(layout, m, n, k, seed):
    """Oracle codes and scales for one layout, as (a, sa, b, sb, sb_n, sb_k, ref64)."""
    if layout == pf8.PF8_WGRAD:
        dyt = _rand_bits((k, m + (-m % 8)), seed, 1e-3, outliers=False)
        xt = _rand_bits((k, n + (-n % 8)), seed + 1)
        qa, sa = oracle.quant_act_1x128(dyt, "rows")
        qb, sb = oracle.quant_act_1x128(xt, "rows")
        ref = oracle.gemm_wgrad(qa[:m], sa[:, :m], qb[:n], sb[:, :n])
        return qa[:m], sa, qb[:n], sb, 1, sb.shape[1], ref
    n_pad = (n + 127) // 128 * 128
    if layout == pf8.PF8_FPROP:
        qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), seed), "cols")
        qw, _, sw = oracle.quant_w_128x128(_rand_bits((n_pad, k), seed + 1, 0.02, outliers=False))
        return qa, sa, qw[:n], sw, sw.shape[1], 1, oracle.gemm_fprop(qa, sa, qw[:n], sw)
    qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), seed, 1e-3, outliers=False), "cols")
    _, qwt, sw = oracle.quant_w_128x128(_rand_bits((k, n_pad), seed + 1, 0.01, outliers=False))
    return qa, sa, qwt[:n], sw, 1, sw.shape[1], oracle.gemm_dgrad(qa, sa, qwt[:n], sw)


LAYOUTS = {"fprop": pf8.PF8_FPROP, "dgrad": pf8.PF8_DGRAD, "wgrad": pf8.PF8_WGRAD}


@pytest.mark.parametrize("lname", list(LAYOUTS))
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 130, 256), (257, 129, 384), (640, 448, 256), (2050, 5407, 384),
                                   (1024, 1024, 640)])
def test_gemm_f32_matches_oracle_and_bf16_path(lname, m, n, k):
    layout = LAYOUTS[lname]
    qa, sa, qb, sb, sb_n, sb_k, ref = _operands(layout, m, n, k, m + 3 * n + k)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k, variant=pf8.PF8_GEMM_MX_SCALED)
    torch.cuda.synchronize()
    got = d32.cpu().numpy().astype(np.float64)
    rep = oracle.gemm_tolerance_report(got, ref)  # (its BF16 bit-equality diagnostic is for BF16 outputs)
    assert rep["violations"] == 0, f"f32 {lname} {m}x{n}x{k}: {rep}"
    # the BF16 kernels hold the same FP32 accumulators: rounding the FP32 result reproduces them
    assert np.array_equal(oracle.bf16_round_from_f64(got), bf16_bits(d16))


@pytest.mark.parametrize("lname", ["fprop", "dgrad"])
def test_gemm_many_rounds_matches_f32_path_and_oracle(lname):
    """A launch of four rounds of 256x256 tiles on 256 CUs (16 x 64 = 1024 tiles, K = 384): every
    output must equal the rounded result of the FP32 kernel, and sampled rows (the first and last
    included) must meet the oracle's tolerance."""
    layout = LAYOUTS[lname]
    m, n, k = 4096, 16384, 384
    if layout == pf8.PF8_FPROP:
        qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), 91), "cols")
        qb, _, sb = oracle.quant_w_128x128(_rand_bits((n, k), 92, 0.02, outliers=False))
        sb_n, sb_k = sb.shape[1], 1
        ref_rows = lambda r: oracle.gemm_fprop(qa[r], sa[:, r], qb, sb)  # noqa: E731
    else:
        qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), 93, 1e-3, outliers=False), "cols")
        _, qb, sb = oracle.quant_w_128x128(_rand_bits((k, n), 94, 0.01, outliers=False))
        sb_n, sb_k = 1, sb.shape[1]
        ref_rows = lambda r: oracle.gemm_dgrad(qa[r], sa[:, r], qb, sb)  # noqa: E731
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    torch.cuda.synchronize()
    assert torch.equal(d32.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    rows = np.concatenate([[0], np.sort(np.random.default_rng(95).choice(m - 2, 62, replace=False) + 1), [m - 1]])
    got = bf16_f64(d16[torch.from_numpy(rows).to(DEV)])
    rep = oracle.gemm_tolerance_report(got, ref_rows(rows))
    assert rep["violations"] == 0, f"{lname}: {rep}"


@pytest.mark.parametrize("lname", list(LAYOUTS))
def test_ragged_tiles_in_odd_rounds(lname):
    """3000 x 8200 in 256x256 tiles is 12 x 33 = 396 tiles, 49 or 50 per XCD: the second round of
    each XCD walks K from its end, and it holds ragged tiles (M edge, and the corner tile with both
    edges). The BF16 result equals the rounded FP32 kernel's (same tiles, same rounds) and meets the
    oracle's bar on every column of sampled rows, the last row included."""
    layout = LAYOUTS[lname]
    m, n, k = 3000, 8200, 1024
    qa, sa, qb, sb, sb_n, sb_k, ref = _operands(layout, m, n, k, 7 * m + n)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    torch.cuda.synchronize()
    assert torch.equal(d32.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    rows = np.unique(np.concatenate([[0, 2815, 2816, m - 1], _sample_rows(m, 60, m + k)]))
    _report(bf16_f64(d16[torch.from_numpy(rows).to(DEV)]), ref[rows], f"{lname} {m}x{n}x{k}")


# One ragged (M, N) per macro-tile the launcher picks (128x128, 256x128, 256x192, 192x256,
# 256x256), and K values whose stage counts (K/64 = 8, 12, 14) give the K loop's head lengths
# 3, 7 and 9 (the shapes above cover 1 and 5, and the two-buffer pipeline).
HEAD_TILES = [(300, 200), (644, 5407), (1421, 5407), (2050, 5407), (2309, 4874)]


def _codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0  # no NaN codes
    return q


@pytest.mark.parametrize("lname", list(LAYOUTS))
@pytest.mark.parametrize("k", [512, 768, 896])
@pytest.mark.parametrize("mn", HEAD_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
def test_every_tile_shape_and_head_length(mn, k, lname):
    """Random E4M3 codes (every finite code, so both operands are heavy-tailed) with power-of-two
    scales per block; sampled output rows (first and last included) against the oracle, inside
    the accumulation contract."""
    m, n = mn
    layout = LAYOUTS[lname]
    rng = np.random.default_rng(m * 31 + n * 7 + k + layout)
    qa, qb = _codes(rng, (m, k)), _codes(rng, (n, k))
    pow2 = lambda *sh: np.ldexp(1.0, rng.integers(-6, 7, size=sh)).astype(np.float32)  # noqa: E731
    sa = pow2(k // 128, m)
    nt = (n + 127) // 128
    if layout == pf8.PF8_FPROP:
        sb, sb_n, sb_k = pow2(nt, k // 128), k // 128, 1
        ref_rows = lambda r: oracle.gemm_fprop(qa[r], sa[:, r], qb, sb)  # noqa: E731
        deq_b = oracle.dequant_w_tiles(qb, sb)
    elif layout == pf8.PF8_DGRAD:
        sb, sb_n, sb_k = pow2(k // 128, nt), 1, nt  # W's tile grid read with swapped strides
        ref_rows = lambda r: oracle.gemm_dgrad(qa[r], sa[:, r], qb, sb)  # noqa: E731
        deq_b = oracle.dequant_w_tiles(qb, sb.T)
    else:
        sb, sb_n, sb_k = pow2(k // 128, n), 1, n
        ref_rows = lambda r: oracle.gemm_wgrad(qa[r], sa[:, r], qb, sb)  # noqa: E731
        deq_b = oracle.dequant_act_groups(qb, sb)
    d = pf8.block_gemm(layout, to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb), sb_n, sb_k)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(k).choice(m, min(m, 48), replace=False)]))
    got = bf16_f64(d[torch.from_numpy(rows).to(DEV)])
    _contract(got, ref_rows(rows), oracle.dequant_act_groups(qa[rows], sa[:, rows]), deq_b, f"{lname} {m}x{n}x{k}")


@pytest.mark.parametrize("lname", ["wgrad", "fprop"])
def test_gemm_f32_accumulates_into_output(lname):
    layout = LAYOUTS[lname]
    m, n, k = 384, 520, 512
    qa, sa, qb, sb, sb_n, sb_k, _ = _operands(layout, m, n, k, 77)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    prod = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    g = torch.Generator(device="cpu").manual_seed(5)
    base = torch.randn((m, n + 4), generator=g).to(DEV)[:, :n]  # padded pitch, 16-byte rows
    pad_before = base.as_strided((m, 4), (n + 4, 1), n).clone()
    start = base.clone()
    pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k, out=base, accumulate=True)
    pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k, out=base, accumulate=True)
    torch.cuda.synchronize()
    # two accumulations: ((start + p) + p) in FP32, element by element
    assert torch.equal(base, (start + prod) + prod)
    assert torch.equal(base.as_strided((m, 4), (n + 4, 1), n), pad_before)  # padding untouched


def test_gemm_f32_validation_on_device():
    a = torch.zeros((128, 128), dtype=torch.uint8, device=DEV)
    s = torch.ones((1, 128), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    d = torch.zeros((128, 128), dtype=torch.float32, device=DEV)
    args = (pf8.PF8_WGRAD, 128, 128, 128, a.data_ptr(), 128, s.data_ptr(), 128, a.data_ptr(), 128, s.data_ptr(), 1,
            128, d.data_ptr(), 128)
    assert pf8.pf8_block_gemm_f32(*args, 2, st) == pf8._lib.PF8_EINVAL
    assert pf8.pf8_block_gemm_f32(*args[:-1], 130, 0, st) == pf8._lib.PF8_EALIGN  # 520-byte pitch
    assert pf8.pf8_block_gemm_f32(*args, 0, st) == pf8._lib.PF8_OK
    torch.cuda.synchronize()
    assert torch.count_nonzero(d) == 0


def test_wrappers_refuse_scale_tensors_too_small():
    """The Python wrappers check the scale tensors' extents before enqueueing anything."""
    a = torch.zeros((256, 256), dtype=torch.uint8, device=DEV)
    sa, sw = torch.ones((2, 256), device=DEV), torch.ones((2, 2), device=DEV)
    with pytest.raises(ValueError, match="b_dscale"):
        pf8.fprop(a, sa, a, torch.ones((1, 2), device=DEV))       # one tile row of W's scales for two
    with pytest.raises(ValueError, match="a_dscale"):
        pf8.fprop(a, sa[:1], a, sw)                               # one K block of X's scales for two
    with pytest.raises(ValueError, match="b_dscale"):
        pf8.wgrad_f32(a, sa, a, torch.ones((2, 255), device=DEV))  # a column of X's scales short
    y = pf8.fprop(a, sa, a, sw)                    # the right sizes still run
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


# ---- plain BF16 GEMM (comparison kernel) against float64 A . B^T ----

@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 130, 256), (257, 129, 384), (640, 448, 2048), (2309, 1000, 640),
                                   (512, 512, 128)])
def test_gemm_bf16_matches_definition(m, n, k):
    ab = _rand_bits((m, k), m + k)
    bb = _rand_bits((n, k), n + 2 * k, 0.02, outliers=False)
    d = pf8.gemm_bf16(to_dev_bf16(ab), to_dev_bf16(bb))
    torch.cuda.synchronize()
    _report(bf16_f64(d), oracle.unquantized_reference(ab, bb), f"bf16 {m}x{n}x{k}")


def test_gemm_bf16_small_integers_exact():
    rng = np.random.default_rng(8)
    for m, n, k in [(64, 64, 128), (300, 260, 1024)]:
        a = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
        b = rng.integers(-4, 5, size=(n, k)).astype(np.float32)
        ab, bb = f32_to_bf16_bits(a), f32_to_bf16_bits(b)
        d = pf8.gemm_bf16(to_dev_bf16(ab), to_dev_bf16(bb))
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(d), oracle.bf16_round_from_f64(oracle.unquantized_reference(ab, bb)))


def test_gemm_bf16_padded_pitches():
    m, n, k = 300, 200, 384
    ab = _rand_bits((m, k), 91)
    bb = _rand_bits((n, k), 92, 0.02, outliers=False)
    abig = np.zeros((m, k + 64), np.uint16)
    abig[:, :k] = ab
    bbig = np.zeros((n, k + 128), np.uint16)
    bbig[:, :k] = bb
    canary = 0x7F80
    d = torch.full((m, 208), 0, dtype=torch.int16, device=DEV).fill_(canary).view(torch.bfloat16)
    a_d, b_d = to_dev_bf16(abig), to_dev_bf16(bbig)
    pf8._lib.check(pf8.pf8_gemm_bf16(m, n, k, a_d.data_ptr(), k + 64, b_d.data_ptr(), k + 128, d.data_ptr(), 208,
                                     torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    bits = bf16_bits(d)
    assert np.all(bits[:, n:] == canary)
    _report((bits[:, :n].astype(np.uint32) << 16).view(np.float32).astype(np.float64),
            oracle.unquantized_reference(ab, bb), "bf16 padded")


def test_full_size_bf16_and_f32_gemms_sampled():
    """The comparison BF16 GEMM on the fprop shape and the FP32 weight gradient accumulated into a
    main gradient on the layer step's wgrad shape, at full size, on sampled output rows."""
    rng = np.random.default_rng(61)
    m, n, k = 8192, 12288, 2048
    ab = f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    bb = f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    d = pf8.gemm_bf16(to_dev_bf16(ab), to_dev_bf16(bb))
    torch.cuda.synchronize()
    rows = _sample_rows(m, 96, 62)
    _report(bf16_f64(d)[rows], oracle.unquantized_reference(ab[rows], bb), "bf16 8192x12288x2048")
    del d
    # wgrad of the layer step: dW [12288, 2048] = dY^T X over 8192 tokens, FP32, accumulated twice
    t = generate("mlp_gateup_layer_step", only=["X", "dY"])
    qdyt, sdyt = pf8.quant_act_1x128(to_dev_bf16(t["dY"]), "rows")
    qxt, sxt = pf8.quant_act_1x128(to_dev_bf16(t["X"]), "rows")
    base = torch.full((12288, 2048), 0.25, dtype=torch.float32, device=DEV)
    pf8.wgrad_f32(qdyt, sdyt, qxt, sxt, out=base, accumulate=True)
    pf8.wgrad_f32(qdyt, sdyt, qxt, sxt, out=base, accumulate=True)
    torch.cuda.synchronize()
    cols = _sample_rows(12288, 96, 63)
    r_qdyt, r_sdyt = oracle.quant_act_1x128(np.ascontiguousarray(t["dY"][:, cols]), "rows")
    r_qxt, r_sxt = oracle.quant_act_1x128(t["X"], "rows")
    ref = 0.25 + 2.0 * oracle.gemm_wgrad(r_qdyt, r_sdyt, r_qxt, r_sxt)
    got = base.cpu().numpy()[cols].astype(np.float64)
    rep = oracle.gemm_tolerance_report(got, ref)
    assert rep["violations"] == 0, rep


# ---- persistent kernel: shapes with two tiles or more per CU, K a multiple of 256 ----
# (M, N, K) per layout. The tile-shape model picks the same shape for the BF16 and the FP32 result
# on each of them, and the BF16 result takes the persistent kernel: 256x256 tiles (four, two, and
# 3.97 rounds of one tile per CU, the last with a tile count that is not a multiple of 8) and
# 192x256 tiles, with tile-scaled (fprop, dgrad) and row-scaled (wgrad) B operands.
PERSISTENT = [("fprop", 4096, 16384, 512), ("dgrad", 8192, 4096, 768), ("fprop", 7936, 8448, 1024),
              ("fprop", 4608, 8192, 1024), ("dgrad", 9216, 4096, 768),
              ("wgrad", 12288, 2048, 1024), ("wgrad", 8192, 4096, 1024)]


@pytest.mark.parametrize("lname,m,n,k", PERSISTENT, ids=lambda v: str(v))
def test_persistent_kernel_matches_one_tile_kernel_and_oracle(lname, m, n, k):
    """The persistent kernel sums every element's products in the one-tile kernel's order (K
    backward in the same odd rounds): its BF16 result equals the rounded result of the FP32 kernel
    (one tile per workgroup, same tile shape) bit for bit; sampled rows, the first and last
    included, meet the oracle's bar."""
    layout = LAYOUTS[lname]
    qa, sa, qb, sb, sb_n, sb_k, _ = _operands_nosample(layout, m, n, k, m + n + k)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    torch.cuda.synchronize()
    assert torch.equal(d32.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    rows = np.unique(np.concatenate([[0, m - 1], _sample_rows(m, 48, m + k)]))
    got = bf16_f64(d16[torch.from_numpy(rows).to(DEV)])
    _report(got, _ref_rows(layout, qa, sa, qb, sb, rows), f"{lname} {m}x{n}x{k}")


def _operands_nosample(layout, m, n, k, seed):
    """Workload-distributed codes for one layout (activations with outliers, weights and
    gradients Gaussian), as (a, sa, b, sb, sb_n, sb_k, None)."""
    if layout == pf8.PF8_WGRAD:
        qa, sa = oracle.quant_act_1x128(_rand_bits((k, m), seed, 1e-3, outliers=False), "rows")
        qb, sb = oracle.quant_act_1x128(_rand_bits((k, n), seed + 1), "rows")
        return qa, sa, qb, sb, 1, sb.shape[1], None
    if layout == pf8.PF8_FPROP:
        qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), seed), "cols")
        qw, _, sw = oracle.quant_w_128x128(_rand_bits((n, k), seed + 1, 0.02, outliers=False))
        return qa, sa, qw, sw, sw.shape[1], 1, None
    qa, sa = oracle.quant_act_1x128(_rand_bits((m, k), seed, 1e-3, outliers=False), "cols")
    _, qwt, sw = oracle.quant_w_128x128(_rand_bits((k, n), seed + 1, 0.01, outliers=False))
    return qa, sa, qwt, sw, 1, sw.shape[1], None


def _ref_rows(layout, qa, sa, qb, sb, rows):
    if layout == pf8.PF8_FPROP:
        return oracle.gemm_fprop(qa[rows], sa[:, rows], qb, sb)
    if layout == pf8.PF8_DGRAD:
        return oracle.gemm_dgrad(qa[rows], sa[:, rows], qb, sb)
    return oracle.gemm_wgrad(qa[rows], sa[:, rows], qb, sb)


@pytest.mark.parametrize("lname,m,n,k", [("dgrad", 4096, 8192, 512), ("wgrad", 12288, 2048, 512)], ids=lambda v: str(v))
def test_persistent_kernel_arbitrary_codes_within_contract(lname, m, n, k):
    """Arbitrary E4M3 codes in both operands and power-of-two scales per block through the persistent
    kernel (256x256 and 192x256 tiles): sampled rows inside the accumulation contract, and the same
    bits as the FP32 kernel rounded."""
    layout = LAYOUTS[lname]
    rng = np.random.default_rng(m + n + k)
    qa, qb = _codes(rng, (m, k)), _codes(rng, (n, k))
    pow2 = lambda *sh: np.ldexp(1.0, rng.integers(-6, 7, size=sh)).astype(np.float32)  # noqa: E731
    sa = pow2(k // 128, m)
    if layout == pf8.PF8_DGRAD:
        sb, sb_n, sb_k = pow2(k // 128, n // 128), 1, n // 128
        deq_b = oracle.dequant_w_tiles(qb, sb.T)
    else:
        sb, sb_n, sb_k = pow2(k // 128, n), 1, n
        deq_b = oracle.dequant_act_groups(qb, sb)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    torch.cuda.synchronize()
    assert torch.equal(d32.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    rows = np.unique(np.concatenate([[0, m - 1], _sample_rows(m, 32, k)]))
    got = bf16_f64(d16[torch.from_numpy(rows).to(DEV)])
    _contract(got, _ref_rows(layout, qa, sa, qb, sb, rows), oracle.dequant_act_groups(qa[rows], sa[:, rows]), deq_b,
              f"{lname} {m}x{n}x{k}")


def test_persistent_kernel_repeats_bitwise_between_other_launches():
    """Twenty launches of the persistent kernel, each after other GEMM and quantiser launches that
    reuse the caches and the CUs, give the same bits every time (a wait that counted too few loads
    would read stale LDS operands now and then)."""
    m, n, k = 4096, 8192, 1024
    qa, sa, qb, sb, sb_n, sb_k, _ = _operands_nosample(pf8.PF8_FPROP, m, n, k, 7)
    a, sa_d, b, sb_d = to_dev_u8(qa), to_dev_f32(sa), to_dev_u8(qb), to_dev_f32(sb)
    first = pf8.block_gemm(pf8.PF8_FPROP, a, sa_d, b, sb_d, sb_n, sb_k)
    other_x = to_dev_bf16(_rand_bits((1024, 2048), 8))
    for i in range(20):
        pf8.quant_act_1x128(other_x, "cols")
        pf8.block_gemm(pf8.PF8_FPROP, a[:1000], sa_d, b[:700], sb_d, sb_n, sb_k)  # ragged: one-tile kernel
        again = pf8.block_gemm(pf8.PF8_FPROP, a, sa_d, b, sb_d, sb_n, sb_k)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16)), f"launch {i}"
