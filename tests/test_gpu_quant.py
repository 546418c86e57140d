"""GPU quantisers vs the CPU oracle: codes and scales bit-exact (runs on an MI355X)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_pf8_amd as pf8
import oracle
from workloads import f32_to_bf16_bits, generate
from tests.gpu_helpers import DEV, f32, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def _check_act(bits, along):
    q, s = pf8.quant_act_1x128(to_dev_bf16(bits), along)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_1x128(bits, along)
    gq, gs = u8(q), f32(s)
    assert gq.shape == q_ref.shape and gs.shape == s_ref.shape
    bad = np.count_nonzero(gq != q_ref)
    assert bad == 0, f"{bad} code mismatches, first at {np.argwhere(gq != q_ref)[:5].tolist()}"
    assert np.array_equal(gs.view(np.uint32), s_ref.view(np.uint32))


def _check_w(bits):
    q, qt, s = pf8.quant_w_128x128(to_dev_bf16(bits))
    torch.cuda.synchronize()
    q_ref, qt_ref, s_ref = oracle.quant_w_128x128(bits)
    assert np.array_equal(u8(q), q_ref)
    assert np.array_equal(u8(qt), qt_ref)
    assert np.array_equal(f32(s).view(np.uint32), s_ref.view(np.uint32))


def _every_bf16_pattern(rows_of=512):
    """All finite bf16 patterns, shuffled into rows so each 128-group has a different maximum."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(f)]
    rng = np.random.default_rng(0)
    bits = rng.permutation(bits)
    n = (len(bits) // rows_of) * rows_of
    return bits[:n].reshape(-1, rows_of)


def test_row_mode_every_bf16_pattern():
    _check_act(_every_bf16_pattern(512), "cols")


def test_col_mode_every_bf16_pattern():
    b = _every_bf16_pattern(512)  # [127, 512] -> take 128 rows x 512 worth by tiling
    b = np.concatenate([b, b[:1]], 0)[:128]
    _check_act(np.ascontiguousarray(b), "rows")
    _check_act(np.ascontiguousarray(b[:, ::-1]), "rows")


def test_weight_every_bf16_pattern():
    b = _every_bf16_pattern(128)[:384]
    _check_w(np.ascontiguousarray(b.reshape(384, 128)))


def test_special_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 512)) * 0.3).astype(np.float32)
    x[0, :128] = 0.0                        # all-zero group -> e = 0
    x[1, :128] = -0.0                       # negative zeros keep their sign
    x[2, :128] = np.float32(2.0 ** -133)    # smallest subnormal: clamp e = -126
    x[3, :128] = np.float32(-3.3895314e38)  # largest finite bf16 magnitude: e = 120
    x[4, 128:256] = np.float32(448.0)       # exactly 448 * 2^0
    x[5, 128:256] = 450.0                   # just above: e = 1
    x[6, 256:384] *= np.float32(1e-30)
    x[7, :] = np.float32(2.0 ** -140)       # rounds to bf16 zero / tiny
    bits = f32_to_bf16_bits(x)
    _check_act(bits, "cols")
    _check_act(bits, "rows")
    _check_w(bits)


@pytest.mark.parametrize("key,name", [("tiny_fprop", "X"), ("attn_fprop", "X"), ("mlp_down_fprop_dgrad", "X"),
                                      ("mlp_down_fprop_dgrad", "dY")])
def test_row_mode_workloads(key, name):
    _check_act(generate(key, only=[name])[name], "cols")


@pytest.mark.parametrize("key,name", [("wgrad", "dY"), ("wgrad", "X"), ("tiny_fprop", "X")])
def test_col_mode_workloads(key, name):
    _check_act(generate(key, only=[name])[name], "rows")


@pytest.mark.parametrize("key", ["tiny_fprop", "attn_fprop", "mlp_gateup_fprop", "mlp_down_fprop_dgrad"])
def test_weight_workloads(key):
    _check_w(generate(key, only=["W"])["W"])


@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 256), (63, 128), (65, 384), (1000, 640)])
def test_row_mode_ragged_rows(rows, cols):
    rng = np.random.default_rng(rows)
    _check_act(f32_to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32)), "cols")


@pytest.mark.parametrize("rows,cols", [(128, 8), (128, 72), (256, 136), (384, 2056)])
def test_col_mode_ragged_cols(rows, cols):
    rng = np.random.default_rng(cols)
    _check_act(f32_to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32)), "rows")


def test_strided_inputs_and_untouched_padding():
    """Leading dimensions larger than the rows: padding bytes of q and dscale stay untouched."""
    rng = np.random.default_rng(9)
    bits = f32_to_bf16_bits(rng.standard_normal((200, 384)).astype(np.float32))
    big = np.zeros((200, 512), np.uint16)
    big[:, :384] = bits
    x = to_dev_bf16(big)[:, :384]
    q = torch.full((200, 400), 0xA5, dtype=torch.uint8, device=DEV)
    s = torch.full((3, 208), -7.0, dtype=torch.float32, device=DEV)
    pf8._lib.check(pf8.pf8_quant_act_1x128(x.data_ptr(), 200, 384, 512, pf8.PF8_ALONG_COLS, q.data_ptr(), 400,
                                           s.data_ptr(), 208, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_1x128(bits, "cols")
    gq, gs = u8(q), f32(s)
    assert np.array_equal(gq[:, :384], q_ref) and np.all(gq[:, 384:] == 0xA5)
    assert np.array_equal(gs[:, :200], s_ref) and np.all(gs[:, 200:] == -7.0)
    # weights with padded pitches, transposed copy too
    wb = f32_to_bf16_bits((rng.standard_normal((256, 384)) * 0.02).astype(np.float32))
    wbig = np.zeros((256, 400), np.uint16)
    wbig[:, :384] = wb
    w = to_dev_bf16(wbig)
    qw = torch.full((256, 400), 0x5A, dtype=torch.uint8, device=DEV)
    qwt = torch.full((384, 272), 0x5A, dtype=torch.uint8, device=DEV)
    sw = torch.full((2, 5), -1.0, dtype=torch.float32, device=DEV)
    pf8._lib.check(pf8.pf8_quant_w_128x128(w.data_ptr(), 256, 384, 400, qw.data_ptr(), 400, qwt.data_ptr(), 272,
                                           sw.data_ptr(), 5, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    q_ref, qt_ref, s_ref = oracle.quant_w_128x128(wb)
    assert np.array_equal(u8(qw)[:, :384], q_ref) and np.all(u8(qw)[:, 384:] == 0x5A)
    assert np.array_equal(u8(qwt)[:, :256], qt_ref) and np.all(u8(qwt)[:, 256:] == 0x5A)
    assert np.array_equal(f32(sw)[:, :3], s_ref) and np.all(f32(sw)[:, 3:] == -1.0)


def test_repeat_runs_are_bitwise_identical():
    bits = generate("tiny_fprop", only=["X"])["X"]
    x = to_dev_bf16(bits)
    a = [pf8.quant_act_1x128(x, "rows") for _ in range(3)]
    torch.cuda.synchronize()
    for q, s in a[1:]:
        assert torch.equal(q, a[0][0]) and torch.equal(s, a[0][1])


# ---- dual-orientation quantiser: one read, both groupings, bit-identical to the two passes ----

def _check_dual(bits):
    qr, sr, qc, sc = pf8.quant_act_dual(to_dev_bf16(bits))
    torch.cuda.synchronize()
    qr_ref, sr_ref = oracle.quant_act_1x128(bits, "cols")
    qc_ref, sc_ref = oracle.quant_act_1x128(bits, "rows")
    for got, ref, what in ((u8(qr), qr_ref, "row codes"), (u8(qc), qc_ref, "col codes")):
        assert got.shape == ref.shape, what
        bad = np.count_nonzero(got != ref)
        assert bad == 0, f"{what}: {bad} mismatches, first at {np.argwhere(got != ref)[:5].tolist()}"
    assert np.array_equal(f32(sr).view(np.uint32), sr_ref.view(np.uint32))
    assert np.array_equal(f32(sc).view(np.uint32), sc_ref.view(np.uint32))


def test_dual_every_bf16_pattern():
    b = _every_bf16_pattern(512)
    b = np.concatenate([b, b[:1]], 0)[:128]
    _check_dual(np.ascontiguousarray(b))
    _check_dual(np.ascontiguousarray(b.reshape(256, 256)[:, ::-1]))


def test_dual_special_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 512)) * 0.3).astype(np.float32)
    x[0, :128] = 0.0
    x[1, :128] = -0.0
    x[:128, 200] = 0.0                      # an all-zero column group
    x[128:, 300] = -0.0
    x[2, :128] = np.float32(2.0 ** -133)
    x[3, :128] = np.float32(-3.3895314e38)
    x[:128, 400] = np.float32(448.0)
    x[128:, 401] = 450.0
    x[6, 256:384] *= np.float32(1e-30)
    x[7, :] = np.float32(2.0 ** -140)
    _check_dual(f32_to_bf16_bits(x))


@pytest.mark.parametrize("key,name", [("tiny_fprop", "X"), ("wgrad", "dY"), ("mlp_gateup_layer_step", "X")])
def test_dual_workloads(key, name):
    _check_dual(generate(key, only=[name])[name])


@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 256), (256, 1152)])
def test_dual_matches_single_orientation_kernels(rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = to_dev_bf16(f32_to_bf16_bits((rng.standard_normal((rows, cols)) * 5).astype(np.float32)))
    qr, sr, qc, sc = pf8.quant_act_dual(x)
    qr1, sr1 = pf8.quant_act_1x128(x, "cols")
    qc1, sc1 = pf8.quant_act_1x128(x, "rows")
    torch.cuda.synchronize()
    assert torch.equal(qr, qr1) and torch.equal(qc, qc1)
    assert torch.equal(sr.view(torch.int32), sr1.view(torch.int32))
    assert torch.equal(sc.view(torch.int32), sc1.view(torch.int32))


def test_dual_strided_inputs_and_untouched_padding():
    rng = np.random.default_rng(11)
    bits = f32_to_bf16_bits(rng.standard_normal((256, 384)).astype(np.float32))
    big = np.zeros((256, 520), np.uint16)
    big[:, :384] = bits
    x = to_dev_bf16(big)[:, :384]
    qr = torch.full((256, 400), 0xA5, dtype=torch.uint8, device=DEV)
    sr = torch.full((3, 264), -7.0, dtype=torch.float32, device=DEV)
    qc = torch.full((384, 272), 0x5A, dtype=torch.uint8, device=DEV)
    sc = torch.full((2, 392), -3.0, dtype=torch.float32, device=DEV)
    pf8._lib.check(pf8.pf8_quant_act_dual(x.data_ptr(), 256, 384, 520, qr.data_ptr(), 400, sr.data_ptr(), 264,
                                          qc.data_ptr(), 272, sc.data_ptr(), 392,
                                          torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    qr_ref, sr_ref = oracle.quant_act_1x128(bits, "cols")
    qc_ref, sc_ref = oracle.quant_act_1x128(bits, "rows")
    gqr, gsr, gqc, gsc = u8(qr), f32(sr), u8(qc), f32(sc)
    assert np.array_equal(gqr[:, :384], qr_ref) and np.all(gqr[:, 384:] == 0xA5)
    assert np.array_equal(gsr[:, :256], sr_ref) and np.all(gsr[:, 256:] == -7.0)
    assert np.array_equal(gqc[:, :256], qc_ref) and np.all(gqc[:, 256:] == 0x5A)
    assert np.array_equal(gsc[:, :384], sc_ref) and np.all(gsc[:, 384:] == -3.0)


def test_dual_rejects_ragged_shapes():
    x = torch.zeros((200, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="unsupported shape"):
        pf8.quant_act_dual(x)


@pytest.mark.parametrize("m,n,k", [(128, 128, 128), (256, 384, 512), (1024, 640, 256)])
def test_fwd_quantiser_matches_separate_calls_and_oracle(m, n, k):
    """pf8_quant_fwd: X's dual quantisation and W's tile quantisation in one launch."""
    rng = np.random.default_rng(m + n + k)
    xb = f32_to_bf16_bits((rng.standard_normal((m, k)) * 2).astype(np.float32))
    wb = f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    e = lambda *sh, dt=torch.uint8: torch.full(sh, 0x77, dtype=dt, device=DEV)  # noqa: E731
    qx, sx, qxt, sxt = e(m, k), e(k // 128, m, dt=torch.float32), e(k, m), e(m // 128, k, dt=torch.float32)
    qw, qwt, sw = e(n, k), e(k, n), e(n // 128, k // 128, dt=torch.float32)
    pf8._lib.check(pf8.pf8_quant_fwd(x.data_ptr(), m, k, k, qx.data_ptr(), k, sx.data_ptr(), m, qxt.data_ptr(), m,
                                     sxt.data_ptr(), k, w.data_ptr(), n, k, qw.data_ptr(), k, qwt.data_ptr(), n,
                                     sw.data_ptr(), k // 128, torch.cuda.current_stream().cuda_stream))
    r_qx, r_sx, r_qxt, r_sxt = pf8.quant_act_dual(x)
    r_qw, r_qwt, r_sw = pf8.quant_w_128x128(w)
    torch.cuda.synchronize()
    for got, want in ((qx, r_qx), (qxt, r_qxt), (qw, r_qw), (qwt, r_qwt)):
        assert torch.equal(got, want)
    for got, want in ((sx, r_sx), (sxt, r_sxt), (sw, r_sw)):
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    o_qx, o_sx = oracle.quant_act_1x128(xb, "cols")
    o_qw, o_qwt, o_sw = oracle.quant_w_128x128(wb)
    assert np.array_equal(u8(qx), o_qx) and np.array_equal(f32(sx), o_sx)
    assert np.array_equal(u8(qw), o_qw) and np.array_equal(u8(qwt), o_qwt) and np.array_equal(f32(sw), o_sw)
