"""The library at its largest accepted sizes, against the oracle (GPU).

- GEMM: K at the largest row pitch whose 256-row tile offsets fit a signed 32-bit offset
  (8,388,480 bytes of codes per row). Small ragged M and N put it on one edge tile, and all
  65,535 K blocks carry their own scales. Compared element by element with the oracle, for
  FP32 and BF16 results.
- GEMM output rows so far apart that a 256-row tile spans more than 2 GB: the kernels' buffer
  stores do not apply and plain 64-bit addresses take over.
- Quantisers: 65,535 grid rows of 128-groups, i.e. the largest grouped dimension each kernel
  accepts. The row-mode case is compared in full. The 2 GB cases are compared on sampled
  128-row bands, always including the first and the last; bands quantise independently.
Inputs: seeded numpy draws, or, for the 2 GB tensors, torch's seeded device generator. The
sampled bands are copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_pf8_amd as pf8
import oracle
from workloads import f32_to_bf16_bits
from tests.gpu_helpers import DEV, bf16_bits, bf16_f64, f32, to_dev_bf16, to_dev_f32, to_dev_u8, u8

pytestmark = pytest.mark.gpu

G = 128
GMAX = 65535 * G                                 # largest grouped dimension (grid rows of 128-groups)
KMAX = ((1 << 31) - 1) // 256 // G * G           # largest K at a legal row pitch: 8,388,480


def _codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0  # no NaN codes
    return q


def _pow2(rng, shape):
    return np.ldexp(1.0, rng.integers(-8, 9, size=shape)).astype(np.float32)


@pytest.mark.parametrize("lname", ["fprop", "wgrad"])
def test_gemm_at_largest_row_pitch(lname):
    m, n, k = 3, 2, KMAX
    rng = np.random.default_rng(11 if lname == "fprop" else 12)
    qa, qb = _codes(rng, (m, k)), _codes(rng, (n, k))
    sa = _pow2(rng, (k // G, m))
    if lname == "fprop":
        layout, sb = pf8.PF8_FPROP, _pow2(rng, (1, k // G))  # W's tile grid [ceil(N/128), K/128]
        sb_n, sb_k = k // G, 1
        # the tile grid's one row of scales applies to both rows of B; handing it over per row keeps
        # the oracle from expanding a whole 128-row tile of scales over 8.4 M columns
        ref = oracle.dequant_act_groups(qa, sa) @ oracle.dequant_act_groups(qb, np.repeat(sb.T, n, axis=1)).T
    else:
        layout, sb = pf8.PF8_WGRAD, _pow2(rng, (k // G, n))  # one scale per K block and row of B
        sb_n, sb_k = 1, n
        ref = oracle.gemm_wgrad(qa, sa, qb, sb)
    a, b, sa_d, sb_d = to_dev_u8(qa), to_dev_u8(qb), to_dev_f32(sa), to_dev_f32(sb)
    assert a.stride(0) == k and b.stride(0) == k
    d32 = pf8.block_gemm_f32(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    d16 = pf8.block_gemm(layout, a, sa_d, b, sb_d, sb_n, sb_k)
    torch.cuda.synchronize()
    got = d32.cpu().numpy().astype(np.float64)
    rep = oracle.gemm_tolerance_report(got, ref)
    assert rep["violations"] == 0, f"{lname} K={k}: {rep}"
    assert np.array_equal(oracle.bf16_round_from_f64(got), bf16_bits(d16))


def test_row_mode_at_largest_group_count():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, GMAX)) * np.repeat(np.ldexp(1.0, rng.integers(-40, 40, (1, GMAX // G))), G, axis=1)
    xb = f32_to_bf16_bits(x.astype(np.float32))
    q, s = pf8.quant_act_1x128(to_dev_bf16(xb), "cols")
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_act_1x128(xb, "cols")
    assert np.array_equal(u8(q), oq) and np.array_equal(f32(s), os_)


def _bands(count, seed, n_sample=48):
    pick = np.random.default_rng(seed).choice(count - 2, n_sample, replace=False) + 1
    return np.concatenate([[0], np.sort(pick), [count - 1]])


def _device_bf16(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.bfloat16)


def _rows_of(t, bands):
    """Host copy of the 128-row bands `bands` of a device tensor, stacked."""
    return torch.cat([t[b * G:(b + 1) * G] for b in bands]).cpu()


def _cols_of(t, cols):
    """Host copy of the columns `cols` of a device tensor (gathered on the device)."""
    return t[:, torch.from_numpy(cols).to(t.device)].cpu().numpy()


def test_col_mode_at_largest_band_count():
    x = _device_bf16((GMAX, 8), 31)
    q, s = pf8.quant_act_1x128(x, "rows")  # q [8, GMAX] (groups along the rows), s [GMAX/128, 8]
    torch.cuda.synchronize()
    bands = _bands(GMAX // G, 32)
    xb = _rows_of(x, bands).view(torch.int16).numpy().view(np.uint16)
    oq, os_ = oracle.quant_act_1x128(xb, "rows")
    cols = np.concatenate([np.arange(b * G, (b + 1) * G) for b in bands])
    assert np.array_equal(_cols_of(q, cols), oq)
    assert np.array_equal(f32(s)[bands], os_)


def test_dual_at_largest_band_count():
    x = _device_bf16((GMAX, G), 41)
    qr, sr, qc, sc = pf8.quant_act_dual(x)
    torch.cuda.synchronize()
    bands = _bands(GMAX // G, 42)
    xb = _rows_of(x, bands).view(torch.int16).numpy().view(np.uint16)
    rows = np.concatenate([np.arange(b * G, (b + 1) * G) for b in bands])
    oqr, osr = oracle.quant_act_1x128(xb, "cols")
    oqc, osc = oracle.quant_act_1x128(xb, "rows")
    assert np.array_equal(_rows_of(qr, bands).numpy(), oqr)
    assert np.array_equal(_cols_of(sr, rows), osr)
    assert np.array_equal(_cols_of(qc, rows), oqc)
    assert np.array_equal(f32(sc)[bands], osc)


def test_weight_tiles_at_largest_band_count():
    w = _device_bf16((GMAX, G), 51) * 0.02
    q, qt, s = pf8.quant_w_128x128(w, transposed=True)
    torch.cuda.synchronize()
    bands = _bands(GMAX // G, 52)
    wb = _rows_of(w, bands).view(torch.int16).numpy().view(np.uint16)
    rows = np.concatenate([np.arange(b * G, (b + 1) * G) for b in bands])
    oq, oqt, os_ = oracle.quant_w_128x128(wb)
    assert np.array_equal(_rows_of(q, bands).numpy(), oq)
    assert np.array_equal(_cols_of(qt, rows), oqt)
    assert np.array_equal(f32(s)[bands], os_)


def test_row_mode_beyond_2g_elements():
    """Row offsets past 2^31 elements: X [2^22 + 128, 512] (2^31 + 65536 values, 4.3 GB)."""
    rows, cols = (1 << 22) + G, 512
    x = _device_bf16((rows, cols), 61)
    q, s = pf8.quant_act_1x128(x, "cols")
    torch.cuda.synchronize()
    pick = np.concatenate([[0], np.sort(np.random.default_rng(62).choice(rows - 2, 62, replace=False) + 1), [rows - 1]])
    idx = torch.from_numpy(pick).to(DEV)
    xb = x[idx].cpu().view(torch.int16).numpy().view(np.uint16)
    oq, os_ = oracle.quant_act_1x128(xb, "cols")
    assert np.array_equal(q[idx].cpu().numpy(), oq)
    assert np.array_equal(_cols_of(s, pick), os_)


def test_gemm_beyond_2g_operand_elements():
    """A [2^22 + 37, 512] codes (2.1 GB, ragged M) against W tiles [200, 512]; sampled output rows,
    the last tile row included, against the oracle."""
    m, n, k = (1 << 22) + 37, 200, 512
    g = torch.Generator(device=DEV).manual_seed(71)
    a = torch.randint(0, 256, (m, k), generator=g, device=DEV, dtype=torch.uint8)
    a[(a & 0x7F) == 0x7F] = 0  # no NaN codes
    sa = torch.pow(2.0, torch.randint(-8, 9, (k // G, m), generator=g, device=DEV).float())
    rng = np.random.default_rng(72)
    qb, sb = _codes(rng, (n, k)), _pow2(rng, (2, k // G))
    d = pf8.fprop(a, sa, to_dev_u8(qb), to_dev_f32(sb))
    torch.cuda.synchronize()
    pick = np.concatenate([np.sort(rng.choice(m - 64, 64, replace=False)), np.arange(m - 64, m)])
    idx = torch.from_numpy(pick).to(DEV)
    qa_s = a[idx].cpu().numpy()
    sa_s = _cols_of(sa, pick)
    ref = oracle.gemm_fprop(qa_s, sa_s, qb, sb)
    got = bf16_bits(d[idx])
    got64 = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rep = oracle.gemm_tolerance_report(got64, ref)
    assert rep["violations"] == 0, rep


def test_gemm_output_pitch_beyond_buffer_range():
    """A BF16 result whose 256-row tiles span more than 2 GB (row pitch 4,194,432 elements): the
    stores cannot use one buffer range per tile, and both kernels that would (the persistent one,
    which this shape's 512 tiles would take, and the one-tile kernel) fall back to plain 64-bit
    addresses. Sampled rows against the oracle; the padding after each sampled row untouched."""
    m, n, k = 512, 65536, 512
    ldd = (1 << 22) + 128  # 256 * ldd * 2 bytes > 2^31 - 1
    rng = np.random.default_rng(41)
    qa, qb = _codes(rng, (m, k)), _codes(rng, (n, k))
    sa = _pow2(rng, (k // G, m))
    sb = _pow2(rng, (n // G, k // G))  # W's tile grid
    a, b, sa_d, sb_d = to_dev_u8(qa), to_dev_u8(qb), to_dev_f32(sa), to_dev_f32(sb)
    buf = torch.full((m, ldd), -7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[:, :n]
    pf8.block_gemm(pf8.PF8_FPROP, a, sa_d, b, sb_d, sb.shape[1], 1, out=out)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 300, m - 1])
    got = bf16_f64(out[torch.from_numpy(rows).to(DEV)])
    ref = oracle.gemm_fprop(qa[rows], sa[:, rows], qb, sb)
    rep = oracle.gemm_tolerance_report(got, ref)
    assert rep["violations"] == 0, rep
    pad = buf[torch.from_numpy(rows).to(DEV), n:n + 4096].float().cpu().numpy()
    assert np.all(pad == -7.0)
    del buf, out
    torch.cuda.empty_cache()
