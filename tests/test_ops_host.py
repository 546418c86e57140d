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
