"""Host-side layout choices of the Python binding (no GPU needed)."""
import fp8_block_scaled_pf8_amd.ops as ops


def test_code_pitch():
    # odd multiples of 4 KiB get 128 more bytes, every other width is kept
    assert ops.code_pitch(12288) == 12416
    assert ops.code_pitch(4096) == 4224
    assert ops.code_pitch(20480) == 20608
    for cols in (128, 384, 2048, 6144, 8192, 16384):
        assert ops.code_pitch(cols) == cols
    # rows stay 128-byte aligned (the quantisers and the GEMM move whole 128-byte lines)
    for cols in range(128, 65536 + 1, 128):
        p = ops.code_pitch(cols)
        assert p >= cols and p % 128 == 0 and p - cols in (0, 128)


def test_out_pitch():
    # BF16 results: 16-byte rows, 128 more bytes when the row is a multiple of 4 KiB
    assert ops.out_pitch(12288, 2) == 12352
    assert ops.out_pitch(2048, 2) == 2112
    assert ops.out_pitch(384, 2) == 384
    assert ops.out_pitch(5407, 2) == 5408
    # FP32 results
    assert ops.out_pitch(2048, 4) == 2080
    assert ops.out_pitch(384, 4) == 384
    for eb in (2, 4):
        for cols in range(1, 9000, 7):
            p = ops.out_pitch(cols, eb)
            assert p >= cols and (p * eb) % 16 == 0 and (p * eb) % 4096 != 0


def test_fp8_linear_checks_weight_codes_before_any_launch():
    """Weight codes of the wrong shape or type are refused on the host."""
    import pytest
    import torch
    from fp8_block_scaled_pf8_amd.linear import fp8_linear

    n, k = 256, 384
    x = torch.zeros((128, k), dtype=torch.bfloat16)
    w = torch.zeros((n, k), dtype=torch.bfloat16)
    good = (torch.zeros((n, k), dtype=torch.uint8), torch.zeros((k, n), dtype=torch.uint8),
            torch.zeros((n // 128, k // 128), dtype=torch.float32))
    bad = [
        (good[0], good[0], good[2]),                                   # codes where the transpose goes
        (good[0], good[1], torch.zeros((k // 128, n // 128))),         # scale grid transposed
        (good[0].float(), good[1], good[2]),                           # not uint8
        (good[0], good[1], good[2].half()),                            # scales not float32
    ]
    for codes in bad:
        with pytest.raises(ValueError, match="w_codes"):
            fp8_linear(x, w, None, codes)


def test_scale_extents_are_checked_on_the_host():
    """Scale tensors too small for the GEMM's shape and strides are refused before any launch."""
    import pytest
    import torch
    from fp8_block_scaled_pf8_amd import _lib as L

    m, n, k = 300, 200, 384                       # ragged M and N, 3 K blocks
    f = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    sa, sw = f(3, m), f(2, 3)                     # X groups [K/128, M]; W tile grid [ceil(N/128), K/128]
    ops._check_scales(L.PF8_FPROP, m, n, k, sa, sw, sw.stride(0), 1)
    ops._check_scales(L.PF8_DGRAD, m, 3 * 128, 2 * 128, f(2, m), sw, 1, sw.stride(0))  # W^T: grid read transposed
    ops._check_scales(L.PF8_WGRAD, m, n, k, sa, f(3, n), 1, n)
    ops._check_scales(L.PF8_FPROP, m, n, k, sa, f(4, 5)[1:3, 1:4], 5, 1)  # a view: storage runs past it
    bad = [
        (L.PF8_FPROP, sa[:2], sw, 3, 1),           # a_dscale misses a K block
        (L.PF8_FPROP, sa[:, :m - 1], sw, 3, 1),    # a_dscale misses a row
        (L.PF8_FPROP, sa, f(1, 3), 3, 1),          # one tile row of W for two
        (L.PF8_WGRAD, sa, f(3, n - 1), 1, n - 1),  # one column short
        (L.PF8_FPROP, sa, sw, 0, 1),               # a zero stride
    ]
    for layout, a_s, b_s, sb_n, sb_k in bad:
        with pytest.raises(ValueError):
            ops._check_scales(layout, m, n, k, a_s, b_s, sb_n, sb_k)
