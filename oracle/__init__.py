"""CPU oracle for the block-scaled FP8 linear-layer path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``fp8_block_scaled_pf8_amd``) never calls it and must fail loudly when its HIP
library is missing.

Plain, slow and obviously correct: numpy in float64 with exact bit arithmetic
on bf16 patterns. It shares no code with the HIP path; the two only consume the
same bf16 bit patterns from ``workloads``.

What it computes, and where the pages say so (sites of the Puro-2B report,
arXiv 2608.27370):

* E4M3 = 4 exponent bits, 3 mantissa bits
  [paper.rainbus.top summary, 前置知识 "FP8 块级混合精度训练"];
* activations and gradients: one power-of-two scale per 128 values along the
  GEMM reduction dimension; weights: one per 128x128 block; scales are
  computed online per block [same section; same page, 方法步骤详情 step (3);
  ta-paperlens explainer, 打ち手2 "ブロック単位FP8を最初から使う" (report §3.2)];
* forward, data-gradient and weight-gradient GEMMs all take blockwise E4M3
  operands [paperlayer.ai summary, appendix C "Production Training Details",
  bullet "FP8 implementation pipeline"].

Readings where the pages are silent:

* block statistic = exact absolute maximum of the current block;
* scale = smallest power of two 2^e with amax <= 448 * 2^e (never saturates);
  all-zero block -> e = 0; e clamped below at -126;
* E4M3 variant = OCP E4M3FN (max 448, no infinities), round to nearest with
  ties to even, sign kept on zero results;
* GEMM reference = exact dequantised operands multiplied in float64 (the
  FP32 accumulation / BF16 output of the fast path is judged against it with
  a tolerance, see ``oracle.gemm``).

Parity pins (tests marked ``not gpu``): brute-force nearest-code search,
exact-rational exponent rule over every positive bf16 value, scalar-loop
grouping on tiny tensors, hand-derived worked examples under
``tests/golden/``, invariants, exact ``Fraction`` GEMM sums and closed forms
(identity / one-hot / permutation weights). No function here is unpinned.
"""
from .e4m3 import E4M3_MAX, decode_e4m3, encode_e4m3, e4m3_table
from .quant import block_exponent, quant_act_1x128, quant_w_128x128
from .gemm import (
    bf16_round_from_f64,
    dequant_act_groups,
    dequant_w_tiles,
    gemm_fprop,
    gemm_dgrad,
    gemm_wgrad,
    gemm_blockwise_exact,
    unquantized_reference,
    gemm_tolerance_report,
    contract_allowance,
    contract_report,
)

__all__ = [
    "E4M3_MAX",
    "decode_e4m3",
    "encode_e4m3",
    "e4m3_table",
    "block_exponent",
    "quant_act_1x128",
    "quant_w_128x128",
    "bf16_round_from_f64",
    "dequant_act_groups",
    "dequant_w_tiles",
    "gemm_fprop",
    "gemm_dgrad",
    "gemm_wgrad",
    "gemm_blockwise_exact",
    "unquantized_reference",
    "gemm_tolerance_report",
    "contract_allowance",
    "contract_report",
]
