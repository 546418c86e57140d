// Host-side launchers of the libpf8 kernels (called by the C ABI after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf8 {

hipError_t launch_quant_rows(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, int64_t ldq,
                             float* dscale, int64_t ld_s, hipStream_t stream);
hipError_t launch_quant_cols(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, int64_t ldq,
                             float* dscale, int64_t ld_s, hipStream_t stream);
hipError_t launch_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, int64_t ldq_row,
                             float* dscale_row, int64_t ld_sr, void* q_col, int64_t ldq_col, float* dscale_col,
                             int64_t ld_sc, hipStream_t stream);
hipError_t launch_quant_fwd(const void* x, int64_t m, int64_t k, int64_t ldx, void* qx, int64_t ldqx, float* sx,
                            int64_t ld_sx, void* qxt, int64_t ldqxt, float* sxt, int64_t ld_sxt, const void* w,
                            int64_t n, int64_t ldw, void* qw, int64_t ldqw, void* qwt, int64_t ldqwt, float* sw,
                            int64_t ld_sw, hipStream_t stream);
hipError_t launch_quant_w(const void* w, int64_t n, int64_t k, int64_t ldw, void* q, int64_t ldq, void* qt,
                          int64_t ldqt, float* dscale, int64_t ld_s, hipStream_t stream);

struct GemmArgs {
  int64_t m, n, k;
  const uint8_t* a;
  int64_t lda;
  const float* a_dscale;
  int64_t ld_as;
  const uint8_t* b;
  int64_t ldb;
  const float* b_dscale;
  int64_t sb_n, sb_k;
  uint16_t* d;     // BF16 output (when d32 is null)
  int64_t ldd;
  float* d32;      // FP32 output instead of d, or null
  int accumulate;  // with d32: add the product to d32's contents instead of overwriting them
};

// row_b_scale: B's scales are per (K-block, row) (wgrad) instead of per 128x128 tile.
// mx: apply the scales inside the block-scaled MFMA; otherwise promote in FP32 registers.
hipError_t launch_gemm(const GemmArgs& args, bool row_b_scale, bool mx, hipStream_t stream);

// Plain BF16 GEMM D = A . B^T (no scales); args.k, lda, ldb in bytes, a_dscale / b_dscale unused.
hipError_t launch_gemm_bf16(const GemmArgs& args, hipStream_t stream);

}  // namespace pf8
