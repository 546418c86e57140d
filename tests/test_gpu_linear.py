"""The FP8 linear layer under autograd (fp8_linear / Fp8Linear) against the CPU oracle.

Forward Y, and backward dX and dW (BF16, or FP32 accumulated into a main gradient over several
micro-batches), each compared element by element with the oracle's GEMM on the oracle's codes,
to |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_pf8_amd as pf8
import oracle
from workloads import f32_to_bf16_bits
from tests.gpu_helpers import DEV, bf16_f64, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bits(shape, seed, sigma, outliers):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    if outliers:
        x.reshape(-1)[rng.choice(x.size, max(1, x.size // 200), replace=False)] *= 50
    return f32_to_bf16_bits(x)


def _check(gpu, ref, what):
    rep = oracle.gemm_tolerance_report(gpu, ref)
    assert rep["violations"] == 0, f"{what}: {rep}"


def _oracle_layer(xb, wb, dyb):
    qx, sx = oracle.quant_act_1x128(xb, "cols")
    qxt, sxt = oracle.quant_act_1x128(xb, "rows")
    qw, qwt, sw = oracle.quant_w_128x128(wb)
    qdy, sdy = oracle.quant_act_1x128(dyb, "cols")
    qdyt, sdyt = oracle.quant_act_1x128(dyb, "rows")
    return (oracle.gemm_fprop(qx, sx, qw, sw), oracle.gemm_dgrad(qdy, sdy, qwt, sw),
            oracle.gemm_wgrad(qdyt, sdyt, qxt, sxt))


@pytest.mark.parametrize("batch,seq,k,n", [(2, 128, 512, 384), (1, 256, 256, 640)])
def test_fp8_linear_forward_backward(batch, seq, k, n):
    m = batch * seq
    xb = _bits((m, k), 1 + k, 1.0, True)
    wb = _bits((n, k), 2 + n, 0.02, False)
    dyb = _bits((m, n), 3 + m, 1e-3, False)
    x = to_dev_bf16(xb).reshape(batch, seq, k).requires_grad_(True)
    w = to_dev_bf16(wb).requires_grad_(True)
    y = pf8.fp8_linear(x, w)
    assert y.shape == (batch, seq, n) and y.dtype == torch.bfloat16
    y.backward(to_dev_bf16(dyb).reshape(batch, seq, n))
    torch.cuda.synchronize()
    ry, rdx, rdw = _oracle_layer(xb, wb, dyb)
    _check(bf16_f64(y.detach().reshape(m, n)), ry, "Y")
    _check(bf16_f64(x.grad.reshape(m, k)), rdx, "dX")
    _check(bf16_f64(w.grad), rdw, "dW")


def test_fp8_linear_fp32_main_grad_accumulates_micro_batches():
    m, k, n = 256, 384, 512
    layer = pf8.Fp8Linear(k, n, device=DEV, fp32_main_grad=True,
                          weight=to_dev_bf16(_bits((n, k), 7, 0.02, False)))
    wb = _bits((n, k), 7, 0.02, False)
    want = np.zeros((n, k))
    for mb in range(3):
        xb = _bits((m, k), 10 + mb, 1.0, True)
        dyb = _bits((m, n), 20 + mb, 1e-3, False)
        x = to_dev_bf16(xb).requires_grad_(True)
        y = layer(x)
        y.backward(to_dev_bf16(dyb))
        want += _oracle_layer(xb, wb, dyb)[2]
    torch.cuda.synchronize()
    assert layer.weight.grad is None
    got = layer.weight.main_grad.cpu().numpy().astype(np.float64)
    _check(got, want, "FP32 main_grad over 3 micro-batches")


def test_fp8_linear_rejects_ragged_tokens():
    x = torch.zeros((100, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="multiples of 128"):
        pf8.fp8_linear(x, w)


def test_fp8_linear_empty_batch():
    """Zero tokens: an empty Y and dX, no weight gradient, the FP32 main gradient left as it was."""
    w = to_dev_bf16(_bits((256, 384), 41, 0.02, False)).requires_grad_(True)
    x = torch.empty((0, 7, 384), dtype=torch.bfloat16, device=DEV).requires_grad_(True)
    y = pf8.fp8_linear(x, w)
    assert tuple(y.shape) == (0, 7, 256) and y.dtype == torch.bfloat16
    y.sum().backward()
    assert tuple(x.grad.shape) == (0, 7, 384) and w.grad is None
    layer = pf8.Fp8Linear(384, 256, device=DEV, fp32_main_grad=True)
    layer.weight.main_grad.fill_(1.5)
    xe = torch.empty((0, 384), dtype=torch.bfloat16, device=DEV, requires_grad=True)
    layer(xe).sum().backward()
    torch.cuda.synchronize()
    assert bool((layer.weight.main_grad == 1.5).all()) and layer.weight.grad is None


def test_fp8_linear_noncontiguous_input():
    """A transposed-view input, made contiguous by the layer before quantisation."""
    m, k, n = 256, 384, 128
    xb = _bits((k, m), 31, 1.0, True)   # stored transposed: X = xt^T
    wb = _bits((n, k), 32, 0.02, False)
    dyb = _bits((m, n), 33, 1e-3, False)
    xt = to_dev_bf16(xb)
    x = xt.t().requires_grad_(True)     # [m, k] view with strides (1, m)
    w = to_dev_bf16(wb).requires_grad_(True)
    y = pf8.fp8_linear(x, w)
    y.backward(to_dev_bf16(dyb))
    torch.cuda.synchronize()
    x_bits = np.ascontiguousarray(xb.T)
    ry, rdx, rdw = _oracle_layer(x_bits, wb, dyb)
    _check(bf16_f64(y.detach()), ry, "Y")
    _check(bf16_f64(x.grad.contiguous()), rdx, "dX")
    _check(bf16_f64(w.grad), rdw, "dW")


def test_fp8_linear_weight_codes_follow_the_weight():
    """Fp8Linear quantises W once per version: micro-batches share the codes, an optimizer step (an
    in-place update) makes new ones, and so does invalidate_weight_codes() after a .data write.
    Each forward is checked against the oracle on the weight as it then stands."""
    m, k, n = 256, 384, 256
    layer = pf8.Fp8Linear(k, n, device=DEV, weight=to_dev_bf16(_bits((n, k), 51, 0.02, False)))
    opt = torch.optim.SGD(layer.parameters(), lr=0.5)
    xb = _bits((m, k), 52, 1.0, True)
    dyb = _bits((m, n), 53, 1e-3, False)

    def forward_checked(what):
        x = to_dev_bf16(xb).requires_grad_(True)
        y = layer(x)
        torch.cuda.synchronize()
        wb = layer.weight.detach().cpu().view(torch.int16).numpy().view(np.uint16)
        ry = _oracle_layer(xb, wb, dyb)[0]
        _check(bf16_f64(y.detach()), ry, what)
        return y

    y = forward_checked("Y, first micro-batch")
    codes = layer.weight_codes()
    y.backward(to_dev_bf16(dyb))
    forward_checked("Y, second micro-batch")
    assert layer.weight_codes() is codes  # unchanged W: the same codes
    opt.step()
    forward_checked("Y after an optimizer step")
    assert layer.weight_codes() is not codes
    codes = layer.weight_codes()
    layer.weight.data.mul_(0.25)  # invisible to the version counter
    layer.invalidate_weight_codes()
    forward_checked("Y after a .data write and invalidate_weight_codes()")
    assert layer.weight_codes() is not codes


def test_fp8_linear_weight_codes_on_another_stream():
    """Codes made on one stream and used by a forward on another: the second stream waits for them
    (the main stream makes them behind a long sleep, so a side stream that did not wait would read
    unfinished codes), and the result equals the one on the main stream."""
    m, k, n = 256, 384, 256
    layer = pf8.Fp8Linear(k, n, device=DEV, weight=to_dev_bf16(_bits((n, k), 61, 0.02, False)))
    x = to_dev_bf16(_bits((m, k), 62, 1.0, True))
    with torch.no_grad():
        y_main = layer(x)
    torch.cuda.synchronize()
    layer.weight.data.mul_(0.5)
    layer.invalidate_weight_codes()
    side = torch.cuda.Stream()
    torch.cuda._sleep(20_000_000)        # keep the main stream busy before it makes the new codes
    codes = layer.weight_codes()          # enqueued behind the sleep, on the main stream
    with torch.cuda.stream(side):
        with torch.no_grad():
            y_side = layer(x)
        assert layer.weight_codes() is codes
    torch.cuda.synchronize()
    with torch.no_grad():
        y_again = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(y_side, y_again)
    assert not torch.equal(y_side, y_main)
