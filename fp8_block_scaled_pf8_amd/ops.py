"""Tensor-level wrappers over the libpf8 C ABI (PyTorch-ROCm supplies device memory and streams).

Each wrapper validates dtypes/devices, allocates its outputs with torch and forwards raw pointers
to the C entry point of the same purpose; every step of the computation runs in libpf8's HIP
kernels. Codes are ``torch.uint8`` (OCP E4M3FN bit patterns; ``.view(torch.float8_e4m3fn)``
reinterprets them), scales are float32 dequantisation multipliers.

Layouts (reduction dimension contiguous for every GEMM operand):
  quant_act_1x128(x [R, C], along="cols") -> q [R, C],  s [C/128, R]
  quant_act_1x128(x [R, C], along="rows") -> q [C, R],  s [R/128, C]
  quant_w_128x128(w [N, K])               -> q [N, K],  qt [K, N] (optional), s [N/128, K/128]
  fprop(qx, sx, qw, sw)     -> Y  [M, N]   = X . W^T
  dgrad(qdy, sdy, qwt, sw)  -> dX [M, K]   = dY . W      (qwt, sw from quant_w_128x128(W))
  wgrad(qdyt, sdy, qxt, sx) -> dW [N, K]   = dY^T . X    (both from the along="rows" quantiser)
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib as L

GROUP = 128


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_2d(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")


def _span(t: torch.Tensor) -> int:
    """Elements from t's first element to the end of its storage."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _check_scales(layout: int, m: int, n: int, k: int, a_dscale: torch.Tensor, b_dscale: torch.Tensor,
                  sb_n: int, sb_k: int) -> None:
    """Raise unless every scale a block-scaled GEMM reads lies inside a_dscale and b_dscale.

    The C ABI receives bare pointers and strides and cannot check this; a scale tensor too small
    for its strides would be read out of bounds on the device. a_dscale is [K/128, >= M].
    b_dscale is read at (j/128)*sb_n + kb*sb_k (FPROP, DGRAD) or kb*sb_k + j*sb_n (WGRAD) for
    rows j < N of B and K blocks kb < K/128.
    """
    if k <= 0 or k % GROUP or m <= 0 or n <= 0:
        return  # the C ABI rejects these shapes itself
    kb = k // GROUP
    if a_dscale.dim() != 2 or a_dscale.shape[0] < kb or a_dscale.shape[1] < m:
        raise ValueError(f"a_dscale must cover [K/128, M] = [{kb}, {m}], got {tuple(a_dscale.shape)}")
    if sb_n < 1 or sb_k < 1:
        raise ValueError("sb_n and sb_k must be positive")
    if layout == L.PF8_WGRAD:
        last = (kb - 1) * sb_k + (n - 1) * sb_n
    else:
        last = ((n + GROUP - 1) // GROUP - 1) * sb_n + (kb - 1) * sb_k
    if last >= _span(b_dscale):
        raise ValueError(f"b_dscale holds {_span(b_dscale)} scales from its first element, but strides "
                         f"({sb_n}, {sb_k}) reach element {last}")


def code_pitch(cols: int) -> int:
    """Row pitch (bytes) of a buffer of E4M3 codes with `cols` per row. An odd multiple of 4 KiB gets
    128 more bytes. The GEMM reads the same 64-byte column slice of many rows at once, and with such
    a pitch those reads crowd a few memory channels: in the gate+up layer step the data gradient,
    whose operands have 12288-byte rows, takes 170 us with a 12416-byte pitch against 201 us
    without. Even multiples (8192) and 2048 gained nothing from padding and keep their width."""
    return cols + 128 if cols % 4096 == 0 and (cols // 4096) % 2 == 1 else cols


def out_pitch(cols: int, elem_bytes: int) -> int:
    """Row pitch (elements) of a GEMM result with `cols` columns: a multiple of 16 bytes, and 128 bytes
    more when that is a multiple of 4 KiB. A tile's epilogue writes the same column slice of 256 rows
    at once, and with such pitches those writes crowd a few memory channels: in the gate+up layer
    step padded results take fprop from 194.6 to 191.7 us and wgrad from 193.6 to 189.0 us."""
    pitch = (cols * elem_bytes + 15) // 16 * 16 // elem_bytes
    if (pitch * elem_bytes) % 4096 == 0:
        pitch += 128 // elem_bytes
    return pitch


def result_buffer(rows: int, cols: int, dtype: torch.dtype, device) -> torch.Tensor:
    """GEMM result [rows, cols] with the row pitch of out_pitch (a view of a wider buffer)."""
    eb = torch.empty((), dtype=dtype).element_size()
    return torch.empty((rows, out_pitch(cols, eb)), dtype=dtype, device=device)[:, :cols]


def code_buffer(rows: int, cols: int, device) -> torch.Tensor:
    """Buffer for E4M3 codes u8 [rows, cols] with the row pitch of code_pitch (a view when padded)."""
    pitch = code_pitch(cols)
    buf = torch.empty((rows, pitch), dtype=torch.uint8, device=device)
    return buf if pitch == cols else buf[:, :cols]


def quant_act_1x128(x: torch.Tensor, along: str = "cols") -> Tuple[torch.Tensor, torch.Tensor]:
    """1x128 power-of-two E4M3 quantisation of activations / gradients."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if along == "cols":
        axis = L.PF8_ALONG_COLS
        q = code_buffer(rows, cols, x.device)
        s = torch.empty((max(cols // GROUP, 1), rows), dtype=torch.float32, device=x.device)
    elif along == "rows":
        axis = L.PF8_ALONG_ROWS
        q = code_buffer(cols, rows, x.device)
        s = torch.empty((max(rows // GROUP, 1), cols), dtype=torch.float32, device=x.device)
    else:
        raise ValueError("along must be 'cols' or 'rows'")
    L.check(L.pf8_quant_act_1x128(x.data_ptr(), rows, cols, x.stride(0), axis, q.data_ptr(), q.stride(0),
                                  s.data_ptr(), s.stride(0), _stream(x)), "pf8_quant_act_1x128")
    return q, s


def quant_act_dual(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Both 1x128 groupings from one read of x [R, C] (R, C multiples of 128).

    Returns (q_row [R, C], s_row [C/128, R], q_col [C, R], s_col [R/128, C]), bit-identical to
    quant_act_1x128(x, "cols") and quant_act_1x128(x, "rows").
    """
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    e = lambda *sh, dt=torch.uint8: torch.empty(sh, dtype=dt, device=x.device)  # noqa: E731
    qr, sr = code_buffer(rows, cols, x.device), e(max(cols // GROUP, 1), rows, dt=torch.float32)
    qc, sc = code_buffer(cols, rows, x.device), e(max(rows // GROUP, 1), cols, dt=torch.float32)
    L.check(L.pf8_quant_act_dual(x.data_ptr(), rows, cols, x.stride(0), qr.data_ptr(), qr.stride(0), sr.data_ptr(),
                                 sr.stride(0), qc.data_ptr(), qc.stride(0), sc.data_ptr(), sc.stride(0), _stream(x)),
            "pf8_quant_act_dual")
    return qr, sr, qc, sc


def quant_w_128x128(w: torch.Tensor, transposed: bool = True
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """128x128-tile power-of-two E4M3 quantisation of a weight; optionally also the transposed codes."""
    _check_2d(w, torch.bfloat16, "w")
    n, k = w.shape
    q = code_buffer(n, k, w.device)
    qt = code_buffer(k, n, w.device) if transposed else None
    s = torch.empty((max(n // GROUP, 1), max(k // GROUP, 1)), dtype=torch.float32, device=w.device)
    L.check(L.pf8_quant_w_128x128(w.data_ptr(), n, k, w.stride(0), q.data_ptr(), q.stride(0),
                                  qt.data_ptr() if qt is not None else 0, qt.stride(0) if qt is not None else 0,
                                  s.data_ptr(), s.stride(0), _stream(w)), "pf8_quant_w_128x128")
    return q, qt, s


def block_gemm(layout: int, a: torch.Tensor, a_dscale: torch.Tensor, b: torch.Tensor, b_dscale: torch.Tensor,
               sb_n: int, sb_k: int, out: Optional[torch.Tensor] = None, variant: int = L.PF8_GEMM_AUTO
               ) -> torch.Tensor:
    """D[m, n] = sum_k deq(A)[m, k] deq(B)[n, k] in FP32, written as BF16 (see include/pf8.h)."""
    _check_2d(a, torch.uint8, "a")
    _check_2d(b, torch.uint8, "b")
    _check_2d(a_dscale, torch.float32, "a_dscale")
    if b_dscale.dtype != torch.float32 or not b_dscale.is_cuda:
        raise TypeError("b_dscale must be a float32 device tensor")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError(f"reduction dims differ: a {tuple(a.shape)}, b {tuple(b.shape)}")
    _check_scales(layout, m, n, k, a_dscale, b_dscale, sb_n, sb_k)
    if out is None:
        # the C ABI wants 16-byte row pitches: pad the allocation, hand back the [m, n] view
        out = result_buffer(m, n, torch.bfloat16, a.device)
    _check_2d(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    L.check(L.pf8_block_gemm_variant(variant, layout, m, n, k, a.data_ptr(), a.stride(0), a_dscale.data_ptr(),
                                     a_dscale.stride(0), b.data_ptr(), b.stride(0), b_dscale.data_ptr(), sb_n, sb_k,
                                     out.data_ptr(), out.stride(0), _stream(a)), "pf8_block_gemm")
    return out


def block_gemm_f32(layout: int, a: torch.Tensor, a_dscale: torch.Tensor, b: torch.Tensor, b_dscale: torch.Tensor,
                   sb_n: int, sb_k: int, out: Optional[torch.Tensor] = None, accumulate: bool = False
                   ) -> torch.Tensor:
    """D[m, n] (+)= sum_k deq(A)[m, k] deq(B)[n, k] in FP32 (see pf8_block_gemm_f32 in include/pf8.h).

    With ``accumulate`` the product is added to ``out`` (required), otherwise ``out`` is overwritten
    (or allocated)."""
    _check_2d(a, torch.uint8, "a")
    _check_2d(b, torch.uint8, "b")
    _check_2d(a_dscale, torch.float32, "a_dscale")
    if b_dscale.dtype != torch.float32 or not b_dscale.is_cuda:
        raise TypeError("b_dscale must be a float32 device tensor")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError(f"reduction dims differ: a {tuple(a.shape)}, b {tuple(b.shape)}")
    _check_scales(layout, m, n, k, a_dscale, b_dscale, sb_n, sb_k)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an output tensor to add to")
        out = result_buffer(m, n, torch.float32, a.device)
    _check_2d(out, torch.float32, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    L.check(L.pf8_block_gemm_f32(layout, m, n, k, a.data_ptr(), a.stride(0), a_dscale.data_ptr(), a_dscale.stride(0),
                                 b.data_ptr(), b.stride(0), b_dscale.data_ptr(), sb_n, sb_k, out.data_ptr(),
                                 out.stride(0), int(accumulate), _stream(a)), "pf8_block_gemm_f32")
    return out


def gemm_bf16(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """D[m, n] = sum_k A[m, k] B[n, k] on BF16 operands (the BF16 comparison kernel)."""
    _check_2d(a, torch.bfloat16, "a")
    _check_2d(b, torch.bfloat16, "b")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError(f"reduction dims differ: a {tuple(a.shape)}, b {tuple(b.shape)}")
    if out is None:
        out = result_buffer(m, n, torch.bfloat16, a.device)
    _check_2d(out, torch.bfloat16, "out")
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    L.check(L.pf8_gemm_bf16(m, n, k, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0), out.data_ptr(),
                            out.stride(0), _stream(a)), "pf8_gemm_bf16")
    return out


def fprop(qx, sx, qw, sw, out=None, variant: int = L.PF8_GEMM_AUTO) -> torch.Tensor:
    """Y = X . W^T from row-mode X codes and W tile codes."""
    return block_gemm(L.PF8_FPROP, qx, sx, qw, sw, sw.stride(0), 1, out, variant)


def dgrad(qdy, sdy, qwt, sw, out=None, variant: int = L.PF8_GEMM_AUTO) -> torch.Tensor:
    """dX = dY . W from row-mode dY codes (along N), W's transposed codes and W's tile grid."""
    return block_gemm(L.PF8_DGRAD, qdy, sdy, qwt, sw, 1, sw.stride(0), out, variant)


def wgrad(qdyt, sdy, qxt, sx, out=None, variant: int = L.PF8_GEMM_AUTO) -> torch.Tensor:
    """dW = dY^T . X from col-mode (token-grouped) dY and X codes."""
    return block_gemm(L.PF8_WGRAD, qdyt, sdy, qxt, sx, 1, sx.stride(0), out, variant)


def wgrad_f32(qdyt, sdy, qxt, sx, out=None, accumulate: bool = False) -> torch.Tensor:
    """dW = dY^T . X in FP32; with ``accumulate``, dW is added to ``out`` (an FP32 main gradient)."""
    return block_gemm_f32(L.PF8_WGRAD, qdyt, sdy, qxt, sx, 1, sx.stride(0), out, accumulate)


class LinearStep:
    """One linear layer's FP8 training pass at a fixed shape, with every buffer preallocated.

    forward:  X [M, K] -> codes along K (and along M for the weight gradient),
              W [N, K] -> tile codes (+ transposed), Y = X . W^T
    backward: dY [M, N] -> codes along N and along M, dX = dY . W, dW = dY^T . X
    With ``fused`` (the default; needs M, N, K multiples of 128) X and dY are each read once by
    the dual-orientation quantiser, and X's and W's quantisers share one launch: five launches.
    Otherwise each orientation has its own pass: eight launches. ``run`` enqueues them on the
    current stream and allocates nothing. ``run(weight_codes=False)`` is the step of a later
    micro-batch of the same optimizer step: W's codes from an earlier full run are reused, and
    X's dual quantiser runs alone.
    """

    def __init__(self, x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, variant: int = L.PF8_GEMM_AUTO,
                 fused: bool = True):
        for t, name in ((x, "x"), (w, "w"), (dy, "dy")):
            _check_2d(t, torch.bfloat16, name)
        (m, k), (n, k2), (m2, n2) = x.shape, w.shape, dy.shape
        if k != k2 or m != m2 or n != n2:
            raise ValueError("inconsistent shapes for X [M,K], W [N,K], dY [M,N]")
        if fused and (m % GROUP or n % GROUP or k % GROUP):
            raise ValueError("the fused step needs M, N and K to be multiples of 128")
        self.x, self.w, self.dy, self.variant, self.fused = x, w, dy, variant, fused
        self.m, self.n, self.k = m, n, k
        dev = x.device
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        c = lambda r, cols: code_buffer(r, cols, dev)  # noqa: E731
        self.qx, self.sx = c(m, k), e(k // GROUP, m, dt=f32)
        self.qw, self.qwt, self.sw = c(n, k), c(k, n), e(n // GROUP, k // GROUP, dt=f32)
        self.qdy, self.sdy = c(m, n), e(n // GROUP, m, dt=f32)
        self.qdyt, self.sdyt = c(n, m), e(m // GROUP, n, dt=f32)
        self.qxt, self.sxt = c(k, m), e(m // GROUP, k, dt=f32)
        r = lambda rows, cols: result_buffer(rows, cols, bf, dev)  # noqa: E731
        self.y, self.dx, self.dw = r(m, n), r(m, k), r(n, k)

    def flops(self) -> int:
        return 3 * 2 * self.m * self.n * self.k

    def launches(self, weight_codes: bool = True):
        """The step as a list of (name, thunk); each thunk enqueues one kernel and returns its status.
        Without ``weight_codes`` W is not quantised (its codes must come from an earlier run)."""
        st = torch.cuda.current_stream(self.x.device).cuda_stream
        m, n, k, v = self.m, self.n, self.k, self.variant
        x, dy = self.x, self.dy
        # code row pitches (padded where a plain pitch would be a multiple of 4 KiB)
        lqx, lqxt, lqw, lqwt = self.qx.stride(0), self.qxt.stride(0), self.qw.stride(0), self.qwt.stride(0)
        lqdy, lqdyt = self.qdy.stride(0), self.qdyt.stride(0)
        ly, ldx, ldw = self.y.stride(0), self.dx.stride(0), self.dw.stride(0)
        quant_x_rows = ("quant_x_rows", lambda: L.pf8_quant_act_1x128(
            x.data_ptr(), m, k, x.stride(0), L.PF8_ALONG_COLS, self.qx.data_ptr(), lqx, self.sx.data_ptr(), m, st))
        quant_x_cols = ("quant_x_cols", lambda: L.pf8_quant_act_1x128(
            x.data_ptr(), m, k, x.stride(0), L.PF8_ALONG_ROWS, self.qxt.data_ptr(), lqxt, self.sxt.data_ptr(), k, st))
        quant_x_dual = ("quant_x_dual", lambda: L.pf8_quant_act_dual(
            x.data_ptr(), m, k, x.stride(0), self.qx.data_ptr(), lqx, self.sx.data_ptr(), m, self.qxt.data_ptr(), lqxt,
            self.sxt.data_ptr(), k, st))
        quant_fwd = ("quant_x_dual_w_tiles", lambda: L.pf8_quant_fwd(
            x.data_ptr(), m, k, x.stride(0), self.qx.data_ptr(), lqx, self.sx.data_ptr(), m, self.qxt.data_ptr(), lqxt,
            self.sxt.data_ptr(), k, self.w.data_ptr(), n, self.w.stride(0), self.qw.data_ptr(), lqw,
            self.qwt.data_ptr(), lqwt, self.sw.data_ptr(), k // GROUP, st))
        quant_w = ("quant_w_tiles", lambda: L.pf8_quant_w_128x128(
            self.w.data_ptr(), n, k, self.w.stride(0), self.qw.data_ptr(), lqw, self.qwt.data_ptr(), lqwt,
            self.sw.data_ptr(), k // GROUP, st))
        fprop = ("fprop_gemm", lambda: L.pf8_block_gemm_variant(
            v, L.PF8_FPROP, m, n, k, self.qx.data_ptr(), lqx, self.sx.data_ptr(), m, self.qw.data_ptr(), lqw,
            self.sw.data_ptr(), k // GROUP, 1, self.y.data_ptr(), ly, st))
        quant_dy_rows = ("quant_dy_rows", lambda: L.pf8_quant_act_1x128(
            dy.data_ptr(), m, n, dy.stride(0), L.PF8_ALONG_COLS, self.qdy.data_ptr(), lqdy, self.sdy.data_ptr(), m, st))
        quant_dy_cols = ("quant_dy_cols", lambda: L.pf8_quant_act_1x128(
            dy.data_ptr(), m, n, dy.stride(0), L.PF8_ALONG_ROWS, self.qdyt.data_ptr(), lqdyt, self.sdyt.data_ptr(), n, st))
        quant_dy_dual = ("quant_dy_dual", lambda: L.pf8_quant_act_dual(
            dy.data_ptr(), m, n, dy.stride(0), self.qdy.data_ptr(), lqdy, self.sdy.data_ptr(), m, self.qdyt.data_ptr(), lqdyt,
            self.sdyt.data_ptr(), n, st))
        dgrad = ("dgrad_gemm", lambda: L.pf8_block_gemm_variant(
            v, L.PF8_DGRAD, m, k, n, self.qdy.data_ptr(), lqdy, self.sdy.data_ptr(), m, self.qwt.data_ptr(), lqwt,
            self.sw.data_ptr(), 1, k // GROUP, self.dx.data_ptr(), ldx, st))
        wgrad = ("wgrad_gemm", lambda: L.pf8_block_gemm_variant(
            v, L.PF8_WGRAD, n, k, m, self.qdyt.data_ptr(), lqdyt, self.sdyt.data_ptr(), n, self.qxt.data_ptr(), lqxt,
            self.sxt.data_ptr(), 1, k, self.dw.data_ptr(), ldw, st))
        if self.fused:
            return [quant_fwd if weight_codes else quant_x_dual, fprop, quant_dy_dual, dgrad, wgrad]
        return ([quant_x_rows] + ([quant_w] if weight_codes else []) +
                [fprop, quant_dy_rows, dgrad, quant_dy_cols, quant_x_cols, wgrad])

    def run(self, weight_codes: bool = True) -> None:
        for name, launch in self.launches(weight_codes):
            L.check(launch(), name)
