"""Block-scaled FP8 (E4M3) linear-layer quantisers and GEMM for AMD MI355X (gfx950).

The computation lives in libpf8.so (HIP kernels behind a C ABI, include/pf8.h); this package
is its Python binding. Importing it fails when the library has not been built.
"""
from . import _lib
from ._lib import (
    PF8_ALONG_COLS,
    PF8_ALONG_ROWS,
    PF8_DGRAD,
    PF8_FPROP,
    PF8_GEMM_AUTO,
    PF8_GEMM_MX_SCALED,
    PF8_GEMM_PROMOTE,
    PF8_WGRAD,
    pf8_abi_version,
    pf8_block_gemm,
    pf8_block_gemm_f32,
    pf8_block_gemm_variant,
    pf8_gemm_bf16,
    pf8_quant_act_1x128,
    pf8_quant_act_dual,
    pf8_quant_fwd,
    pf8_quant_w_128x128,
    pf8_strerror,
)
from .linear import Fp8Linear, Fp8LinearFunction, fp8_linear
from .ops import (LinearStep, block_gemm, block_gemm_f32, dgrad, fprop, gemm_bf16, quant_act_1x128, quant_act_dual,
                  quant_w_128x128, wgrad, wgrad_f32)

__all__ = [
    "PF8_ALONG_COLS", "PF8_ALONG_ROWS", "PF8_FPROP", "PF8_DGRAD", "PF8_WGRAD",
    "PF8_GEMM_AUTO", "PF8_GEMM_MX_SCALED", "PF8_GEMM_PROMOTE",
    "pf8_abi_version", "pf8_block_gemm", "pf8_block_gemm_f32", "pf8_block_gemm_variant", "pf8_gemm_bf16", "pf8_quant_act_1x128", "pf8_quant_act_dual",
    "pf8_quant_fwd", "pf8_quant_w_128x128", "pf8_strerror",
    "LinearStep", "block_gemm", "block_gemm_f32", "dgrad", "fprop", "gemm_bf16", "quant_act_1x128", "quant_act_dual",
    "quant_w_128x128", "wgrad", "wgrad_f32", "Fp8Linear", "Fp8LinearFunction", "fp8_linear",
]
