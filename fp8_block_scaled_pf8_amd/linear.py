"""FP8 linear layer for PyTorch autograd: every matmul and every quantisation runs in libpf8.

Y = X . W^T with X [..., K] bf16 and W [N, K] bf16 (a torch.nn.Linear weight without bias).

forward:  X -> row-mode codes (groups along K) and col-mode codes (groups along the tokens) in one
          read (pf8_quant_act_dual); W -> 128x128-tile codes and the transposed codes; Y = fprop.
backward: dY -> row-mode codes (along N) and col-mode codes (along the tokens) in one read;
          dX = dgrad(dY codes, W^T codes); dW = wgrad(dY^T codes, X^T codes).
Only codes and scales are saved for the backward pass (1 byte per element plus 1/32 of that).

FP32 weight gradients: given ``main_grad`` (an FP32 [N, K] buffer), the backward pass adds dW to
it in FP32 inside the GEMM's epilogue (pf8_block_gemm_f32 with accumulate = 1), the way gradients
are summed over the micro-batches of an optimizer step, and autograd receives no gradient for W.

Weight codes: W changes only at an optimizer step, so ``Fp8Linear`` quantises it once per weight
version (codes, transposed codes and tile scales) and reuses them for every micro-batch until W is
modified. An in-place update of the parameter (as optimizers do) bumps its version counter. An
update through ``weight.data`` bypasses that counter; call ``invalidate_weight_codes()`` after one.

Tokens (the product of the leading dimensions), N and K must be multiples of 128. Zero tokens give
an empty result and no weight-gradient contribution, without a launch.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import ops

GROUP = 128


def _check_shapes(m: int, n: int, k: int) -> None:
    if m % GROUP or n % GROUP or k % GROUP:
        raise ValueError(f"fp8_linear needs tokens, out_features and in_features to be multiples of 128 "
                         f"(got tokens={m}, out={n}, in={k})")


class Fp8LinearFunction(torch.autograd.Function):
    """Autograd function of the FP8 linear layer (see the module docstring)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, main_grad: Optional[torch.Tensor] = None,
                w_codes: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
        lead = x.shape[:-1]
        k = x.shape[-1]
        x2 = x.reshape(-1, k)
        if x2.stride(1) != 1 or x2.stride(0) % 8:
            x2 = x2.contiguous()
        n = w.shape[0]
        _check_shapes(x2.shape[0], n, k)
        ctx.lead, ctx.k, ctx.main_grad = lead, k, main_grad
        if x2.shape[0] == 0:
            # no tokens: an empty result, and no gradient contribution in the backward pass (the
            # library rejects empty dimensions, so nothing is launched)
            ctx.empty = True
            return x.new_empty((*lead, n))
        ctx.empty = False
        qx, sx, qxt, sxt = ops.quant_act_dual(x2)
        qw, qwt, sw = w_codes if w_codes is not None else ops.quant_w_128x128(w.contiguous(), transposed=True)
        # results handed to the caller are plain contiguous tensors (the library's own workspaces
        # use padded row pitches instead)
        y = ops.fprop(qx, sx, qw, sw, out=torch.empty((x2.shape[0], n), dtype=torch.bfloat16, device=x.device))
        ctx.save_for_backward(qxt, sxt, qwt, sw)
        return y.reshape(*lead, n)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        if ctx.empty:
            dx = dy.new_empty((*ctx.lead, ctx.k), dtype=torch.bfloat16) if ctx.needs_input_grad[0] else None
            return dx, None, None, None
        qxt, sxt, qwt, sw = ctx.saved_tensors
        n = qwt.shape[1]
        dy2 = dy.reshape(-1, n)
        if dy2.dtype != torch.bfloat16:
            dy2 = dy2.to(torch.bfloat16)
        if dy2.stride(1) != 1 or dy2.stride(0) % 8:
            dy2 = dy2.contiguous()
        qdy, sdy, qdyt, sdyt = ops.quant_act_dual(dy2)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = ops.dgrad(qdy, sdy, qwt, sw, out=torch.empty((dy2.shape[0], ctx.k), dtype=torch.bfloat16,
                                                              device=dy2.device)).reshape(*ctx.lead, ctx.k)
        if ctx.main_grad is not None:
            ops.wgrad_f32(qdyt, sdyt, qxt, sxt, out=ctx.main_grad, accumulate=True)
        elif ctx.needs_input_grad[1]:
            dw = ops.wgrad(qdyt, sdyt, qxt, sxt, out=torch.empty((n, ctx.k), dtype=torch.bfloat16, device=dy2.device))
        return dx, dw, None, None


def fp8_linear(x: torch.Tensor, w: torch.Tensor, main_grad: Optional[torch.Tensor] = None,
               w_codes: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None) -> torch.Tensor:
    """Y = X . W^T through libpf8's block-scaled FP8 path, differentiable in X and W.

    Without ``main_grad`` W's gradient is returned to autograd in BF16. With it (FP32, W's shape,
    16-byte row pitch) the backward pass adds dW to ``main_grad`` in FP32 instead. ``w_codes``
    are W's codes, transposed codes and tile scales from ``ops.quant_w_128x128(w, transposed=True)``
    for the current W; without them W is quantised here.
    """
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("fp8_linear takes bfloat16 X and W")
    if main_grad is not None and (main_grad.dtype != torch.float32 or tuple(main_grad.shape) != tuple(w.shape)):
        raise ValueError("main_grad must be a float32 tensor of W's shape")
    if w_codes is not None:
        n, k = w.shape
        qw, qwt, sw = w_codes
        if (tuple(qw.shape) != (n, k) or tuple(qwt.shape) != (k, n) or tuple(sw.shape) != (n // GROUP, k // GROUP)
                or qw.dtype != torch.uint8 or qwt.dtype != torch.uint8 or sw.dtype != torch.float32):
            raise ValueError("w_codes must be (codes [N,K] uint8, transposed codes [K,N] uint8, scales [N/128,K/128] float32)")
    return Fp8LinearFunction.apply(x, w, main_grad, w_codes)


class Fp8Linear(torch.nn.Module):
    """Bias-free linear layer whose three GEMMs run in block-scaled FP8 (weights kept in BF16).

    With ``fp32_main_grad`` the weight carries an FP32 ``main_grad`` buffer that every backward
    pass accumulates into (zero it once per optimizer step); ``weight.grad`` then stays None.
    The weight's codes are made once per weight version and shared by the micro-batches (see the
    module docstring).
    """

    def __init__(self, in_features: int, out_features: int, device=None, fp32_main_grad: bool = False,
                 weight: Optional[torch.Tensor] = None):
        super().__init__()
        if weight is None:
            weight = torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        self.weight = torch.nn.Parameter(weight)
        if fp32_main_grad:
            self.weight.main_grad = torch.zeros(self.weight.shape, dtype=torch.float32, device=self.weight.device)
        self._codes = None
        self._codes_key = None
        self._codes_ready = None  # event recorded on the stream that made the codes
        self._codes_users = set()  # streams the codes were handed to

    def weight_codes(self) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """W's codes, transposed codes and tile scales, made once per version of the weight.

        They are made on the current stream. A later call from another stream makes that stream
        wait for them, and marks them as used there, so that the allocator keeps their memory
        until that stream's work is done even after new codes replace them."""
        w = self.weight
        key = (w.data_ptr(), w._version, tuple(w.shape), w.device)
        cur = torch.cuda.current_stream(w.device)
        if self._codes is None or self._codes_key != key:
            with torch.no_grad():
                self._codes = ops.quant_w_128x128(w.detach().contiguous(), transposed=True)
            self._codes_key = key
            self._codes_ready = torch.cuda.Event()
            self._codes_ready.record(cur)
            self._codes_users = {cur.cuda_stream}
        elif cur.cuda_stream not in self._codes_users:
            cur.wait_event(self._codes_ready)
            for t in self._codes:
                t.record_stream(cur)
            self._codes_users.add(cur.cuda_stream)
        return self._codes

    def invalidate_weight_codes(self) -> None:
        """Forget the cached weight codes (after a change to W that its version counter misses)."""
        self._codes = None
        self._codes_key = None
        self._codes_ready = None
        self._codes_users = set()

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return fp8_linear(x, self.weight, getattr(self.weight, "main_grad", None), self.weight_codes())
