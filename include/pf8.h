/*
 * pf8.h - C ABI of libpf8: block-scaled FP8 (E4M3) linear-layer quantisers and GEMM for AMD MI355X (gfx950).
 *
 * The method [Puro-2B report; paper.rainbus.top summary, section "FP8 块级混合精度训练" and
 * 方法步骤详情 step (3); ta-paperlens explainer, 打ち手2 (report §3.2); paperlayer.ai summary,
 * appendix C "Production Training Details"]: the linear-layer GEMMs of training (forward,
 * data-gradient, weight-gradient) run on E4M3 operands. Activations and gradients carry one
 * power-of-two scale per 128 consecutive values along the GEMM reduction dimension, weights one
 * per 128x128 tile; each scale is computed from its own block at quantisation time. The GEMM
 * accumulates in FP32, applies the product of the two operands' block scales for every 128-wide
 * K block, and writes BF16.
 *
 * Conventions shared by every entry point
 *  - Every pointer is a device pointer (HBM) unless stated otherwise; the caller allocates and
 *    owns all buffers. The library never allocates, frees or synchronises and keeps no global
 *    state: calls are thread-safe and re-entrant.
 *  - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL = the null stream).
 *  - Leading dimensions ("ld") are in elements of the array they describe.
 *  - Every argument is validated on the host before anything is enqueued; on error nothing
 *    runs and the call returns the status. A launch failure is reported as PF8_ELAUNCH.
 *    Only the sizes of buffers are out of the library's sight: each buffer must hold every
 *    element its shape, pitch and strides address (the Python binding checks this for the
 *    tensors it is given); a smaller one is read or written out of bounds on the device.
 *  - Scales are dequantisation multipliers: value = scale * decode(code). The quantisers write
 *    exact powers of two 2^e, e in [-126, 120]; an all-zero block gets scale 1.
 *  - E4M3 is the OCP E4M3FN encoding (bias 7, max 448, no infinities), rounded to nearest-even,
 *    sign kept on zero. Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *  - Sizes: every dimension, leading dimension and scale stride is at most 2^31 - 1; a larger one
 *    is refused with PF8_ESHAPE (no such array fits a GPU's memory).
 *  - Alignment: every code / bf16 array base is 16-byte aligned, and its row pitch
 *    (ld * element size) is a multiple of 16 bytes. Scale arrays are 4-byte aligned.
 *  - Row pitches and speed: a GEMM reads (and its epilogue writes) the same column slice of many
 *    rows at once, and some pitches crowd a few memory channels. Measured on MI355X: code arrays
 *    whose row pitch is an odd multiple of 4 KiB, and results whose row pitch is any multiple of
 *    4 KiB, run faster with 128 more bytes of pitch (the Python binding allocates that way).
 *    Keep every row pitch a multiple of 128 bytes.
 */
#ifndef PF8_H
#define PF8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PF8_ABI_VERSION 5

/* The status, grouping-axis and layout types are plain ints, so that an out-of-range value
   reaches the library intact and is refused with PF8_EINVAL (a C enum parameter need not be
   able to carry such a value). The names below are their only valid values. */
typedef int pf8_status;
typedef int pf8_group_axis;
typedef int pf8_layout;

/* Status codes (pf8_status). */
#define PF8_OK 0
#define PF8_EINVAL 1  /* null pointer, unknown enum value, non-positive dimension, ld too small */
#define PF8_ESHAPE 2  /* a grouped / tiled dimension is not a multiple of 128 (or 8, see below), or a size is too large */
#define PF8_EALIGN 3  /* pointer not 16-byte aligned, or row pitch not a multiple of 16 bytes */
#define PF8_ENODEV 4  /* no usable HIP device (the library loads and validates without one) */
#define PF8_ELAUNCH 5 /* the kernel launch reported an error */

/* Grouping axis of the activation / gradient quantiser (pf8_group_axis). */
#define PF8_ALONG_COLS 0 /* row mode: a group is 128 consecutive elements of one row */
#define PF8_ALONG_ROWS 1 /* col mode: a group is 128 consecutive rows of one column; codes are written transposed */

/* GEMM layouts (pf8_layout). */
#define PF8_FPROP 0 /* Y[M,N]  = X[M,K] . W[N,K]^T       B = W codes, one scale per 128x128 tile      */
#define PF8_DGRAD 1 /* dX[M,K] = dY[M,N] . W[N,K]        B = W^T codes [K,N], W's tile scales via strides */
#define PF8_WGRAD 2 /* dW[N,K] = dY[M,N]^T . X[M,K]      B = X^T codes [K,M], one scale per (128-block, row) */

/* GEMM kernel variants (pf8_block_gemm_variant). */
#define PF8_GEMM_AUTO 0      /* the fastest variant for the shape (what pf8_block_gemm runs) */
#define PF8_GEMM_MX_SCALED 1 /* scales applied inside gfx950's block-scaled FP8 MFMA (E8M0 scale operands) */
#define PF8_GEMM_PROMOTE 2   /* unscaled FP8 MFMA per 128-block, then FP32 scale-and-accumulate in registers */

/*
 * 1x128 activation / gradient quantiser [paper.rainbus.top summary, section "FP8 块级混合精度训练";
 * ta-paperlens explainer, 打ち手2: activations and gradients get one scale per 128 elements along
 * the reduction direction].
 *
 * x: bf16 [rows, cols], row pitch ldx (>= cols).
 * axis = PF8_ALONG_COLS (row mode; e.g. fprop X along K, dgrad dY along N):
 *     requires cols % 128 == 0 (rows arbitrary >= 1).
 *     q:      u8 [rows, cols], row pitch ldq >= cols.
 *     dscale: f32 [cols/128][rows], i.e. dscale[g * ld_s + r] for group g of row r; ld_s >= rows.
 * axis = PF8_ALONG_ROWS (col mode; wgrad dY and X along the token dimension):
 *     requires rows % 128 == 0 and cols % 8 == 0.
 *     q:      u8 [cols, rows] (transposed, so the reduction dim is contiguous), row pitch ldq >= rows.
 *     dscale: f32 [rows/128][cols], i.e. dscale[g * ld_s + c]; ld_s >= cols.
 * Returns PF8_OK, PF8_EINVAL, PF8_ESHAPE, PF8_EALIGN, PF8_ENODEV or PF8_ELAUNCH.
 */
pf8_status pf8_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx, pf8_group_axis axis,
                               void* q, int64_t ldq, float* dscale, int64_t ld_s, void* hip_stream);

/*
 * Dual-orientation 1x128 quantiser [same passages as above; the forward pass needs X grouped
 * along K for Y = X.W^T and along the tokens for dW = dY^T.X, the backward pass dY along N for
 * dX = dY.W and along the tokens for dW]: one read of x yields both groupings.
 *
 * x: bf16 [rows, cols], row pitch ldx >= cols; requires rows % 128 == 0 and cols % 128 == 0.
 * Row mode (groups of 128 along a row), exactly as pf8_quant_act_1x128 with PF8_ALONG_COLS:
 *     q_row: u8 [rows, cols], pitch ldq_row >= cols; dscale_row[g * ld_sr + r], ld_sr >= rows.
 * Col mode (groups of 128 along a column), exactly as pf8_quant_act_1x128 with PF8_ALONG_ROWS:
 *     q_col: u8 [cols, rows] (transposed), pitch ldq_col >= rows; dscale_col[g * ld_sc + c], ld_sc >= cols.
 * The four outputs are bit-identical to those of the two single-orientation calls.
 * Returns PF8_OK, PF8_EINVAL, PF8_ESHAPE, PF8_EALIGN, PF8_ENODEV or PF8_ELAUNCH.
 */
pf8_status pf8_quant_act_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                              void* q_row, int64_t ldq_row, float* dscale_row, int64_t ld_sr,
                              void* q_col, int64_t ldq_col, float* dscale_col, int64_t ld_sc, void* hip_stream);

/*
 * Forward-pass quantisers of one linear layer in one launch [the passages above: X grouped along
 * K and along the tokens, W by 128x128 tiles with its transposed codes for the data gradient]:
 * exactly pf8_quant_act_dual(X) and pf8_quant_w_128x128(W), with one workgroup per 128x128 tile
 * of either tensor.
 *
 * X: bf16 [m, k], pitch ldx; qx/sx and qxt/sxt as q_row/dscale_row and q_col/dscale_col of
 *    pf8_quant_act_dual (qx [m, k], sx[g * ld_sx + r], qxt [k, m], sxt[g * ld_sxt + c]).
 * W: bf16 [n, k], pitch ldw; qw, qwt (may be NULL), sw as q, qt, dscale of pf8_quant_w_128x128.
 * m, n and k must be multiples of 128. The outputs are bit-identical to the two separate calls.
 */
pf8_status pf8_quant_fwd(const void* x, int64_t m, int64_t k, int64_t ldx,
                         void* qx, int64_t ldqx, float* sx, int64_t ld_sx,
                         void* qxt, int64_t ldqxt, float* sxt, int64_t ld_sxt,
                         const void* w, int64_t n, int64_t ldw,
                         void* qw, int64_t ldqw, void* qwt, int64_t ldqwt, float* sw, int64_t ld_sw, void* hip_stream);

/*
 * 128x128 weight-tile quantiser [paper.rainbus.top summary, section "FP8 块级混合精度训练" and
 * 方法步骤详情 step (3): weights get one scale per 128x128 block].
 *
 * w:      bf16 [n, k], row pitch ldw >= k; requires n % 128 == 0 and k % 128 == 0.
 * q:      u8 [n, k], row pitch ldq >= k.
 * qt:     u8 [k, n] (the same codes transposed, for the data-gradient GEMM) or NULL; pitch ldqt >= n.
 * dscale: f32 [n/128][k/128], i.e. dscale[tn * ld_s + tk]; ld_s >= k/128.
 */
pf8_status pf8_quant_w_128x128(const void* w, int64_t n, int64_t k, int64_t ldw, void* q, int64_t ldq,
                               void* qt, int64_t ldqt, float* dscale, int64_t ld_s, void* hip_stream);

/*
 * Block-scaled FP8 GEMM [paperlayer.ai summary, appendix C, bullet "FP8 implementation pipeline":
 * the forward, data-gradient and weight-gradient GEMMs run on blockwise E4M3 operands].
 *
 *   D[i, j] = sum_{kb} sa(kb, i) * sb(kb, j) * sum_{k in block kb} decode(A[i, k]) * decode(B[j, k])
 *
 * with FP32 accumulation and a BF16 (round-to-nearest-even) result.
 *
 * Accumulation contract. On gfx950's FP8 matrix instructions (both variants; measured) the
 * products of each aligned group of 8 consecutive k are exact and are added in a fixed-point
 * window: each is truncated toward zero to a multiple of 2^(E-13), where 2^E <= the group's
 * largest |product| < 2^(E+1). Group sums accumulate in FP32. With ref = the exact sum above and
 * p_k = sa * decode(A[i,k]) * sb * decode(B[j,k]), every element therefore satisfies
 *     |D[i,j] - ref| <= 2^-8 |ref| + (1 + 2^-8) * (7 * 2^-13 * sum_{groups g} max_{k in g} |p_k|
 *                                                  + (k / 4) * 2^-24 * sum_k |p_k|)
 * (window truncation, fewer than k/4 FP32 roundings, BF16 rounding). On operands distributed like
 * training activations with rare outliers against Gaussian weights or gradients, the error also
 * stays within |D[i,j] - ref| <= 2^-7 |ref| + 1e-3 rms(ref) (rms over the whole output), the bar
 * the library is tested to on such data. With outliers in both operands an outlier product can
 * take the low bits of the other seven products of its group, and only the contract holds.
 *
 * Order and repeatability. The FP32 sum of an element runs over K forward or backward, by the
 * position of its output tile in the launch (tiles of odd rounds start at the end of K, where the
 * previous round's reads are still cached). The same call on the same device gives the same bits
 * every time; the same rows inside a GEMM of another shape may differ in the last bits of the
 * FP32 sum, always within the contract. No atomics; no split of K across workgroups.
 *
 * m, n >= 1 (any value), k % 128 == 0.
 * a: u8 [m, k] (pitch lda >= k), reduction dim contiguous.  a_dscale: f32, sa(kb, i) = a_dscale[kb * ld_as + i], ld_as >= m.
 * b: u8 [n, k] (pitch ldb >= k), reduction dim contiguous.  b_dscale: f32, with
 *     layout FPROP / DGRAD (tile scales): sb(kb, j) = b_dscale[(j / 128) * sb_n + kb * sb_k]
 *         (fprop passes W's grid: sb_n = ld_s, sb_k = 1; dgrad passes the same grid transposed:
 *          sb_n = 1, sb_k = ld_s);
 *     layout WGRAD (1x128 row groups):  sb(kb, j) = b_dscale[kb * sb_k + j * sb_n]
 *         (the col-mode quantiser's [K/128][n] array: sb_k = ld_s, sb_n = 1).
 * d: bf16 [m, n], row pitch ldd >= n.
 * The MX-scaled variant needs every scale to be an exact power of two in [2^-127, 2^127] (what the
 * quantisers produce); PF8_GEMM_PROMOTE accepts any finite FP32 scales.
 */
pf8_status pf8_block_gemm(pf8_layout layout, int64_t m, int64_t n, int64_t k,
                          const void* a, int64_t lda, const float* a_dscale, int64_t ld_as,
                          const void* b, int64_t ldb, const float* b_dscale, int64_t sb_n, int64_t sb_k,
                          void* d, int64_t ldd, void* hip_stream);

/* Same as pf8_block_gemm with an explicit kernel variant (PF8_GEMM_*); PF8_EINVAL for an unknown one. */
pf8_status pf8_block_gemm_variant(int variant, pf8_layout layout, int64_t m, int64_t n, int64_t k,
                                  const void* a, int64_t lda, const float* a_dscale, int64_t ld_as,
                                  const void* b, int64_t ldb, const float* b_dscale, int64_t sb_n, int64_t sb_k,
                                  void* d, int64_t ldd, void* hip_stream);

/*
 * Block-scaled FP8 GEMM with an FP32 result [paperlayer.ai summary, appendix C "Production
 * Training Details": gradients are kept in FP32; with several micro-batches per optimizer step
 * the weight gradient is a running FP32 sum]:
 *
 *   accumulate = 0:  D[i, j]  = sum_kb sa(kb, i) * sb(kb, j) * sum_{k in block kb} decode(A[i, k]) * decode(B[j, k])
 *   accumulate = 1:  D[i, j] += (the same sum)
 *
 * Layouts, operands, scales and limits are exactly those of pf8_block_gemm; the product is formed
 * by the MX-scaled kernel with FP32 accumulation and is not rounded to BF16. The accumulation
 * contract of pf8_block_gemm holds for the product without its 2^-8 |ref| (BF16) term; with
 * accumulate = 1 the final FP32 addition rounds once more.
 * d: f32 [m, n], row pitch ldd >= n with ldd * 4 a multiple of 16 bytes, 16-byte aligned base.
 * With accumulate = 1 every element of d is read once and written once by a single thread (no
 * atomics); d must not overlap a or b. accumulate other than 0 or 1 is PF8_EINVAL.
 */
pf8_status pf8_block_gemm_f32(pf8_layout layout, int64_t m, int64_t n, int64_t k,
                              const void* a, int64_t lda, const float* a_dscale, int64_t ld_as,
                              const void* b, int64_t ldb, const float* b_dscale, int64_t sb_n, int64_t sb_k,
                              float* d, int64_t ldd, int accumulate, void* hip_stream);

/*
 * Plain BF16 GEMM, the comparison point for the FP8 path [the pages measure FP8 training against
 * BF16 training of the same model: bit.fan article, "FP8 训练换来 1.36 倍吞吐提升"; paperlayer.ai
 * summary, appendix C]: the same pipeline and tiles as the FP8 kernels, on BF16 operands.
 *
 *   D[i, j] = sum_k A[i, k] * B[j, k]     (FP32 accumulation, BF16 round-to-nearest-even output)
 *
 * a: bf16 [m, k], pitch lda >= k; b: bf16 [n, k], pitch ldb >= k (both K-contiguous, as every
 * operand here); d: bf16 [m, n], pitch ldd >= n. m, n >= 1 (any value), k % 128 == 0.
 * Bases 16-byte aligned, pitches multiples of 16 bytes; lda, ldb <= (2^31 - 1) / 512.
 */
pf8_status pf8_gemm_bf16(int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const void* b, int64_t ldb,
                         void* d, int64_t ldd, void* hip_stream);

/* Static, NUL-terminated description of a status code ("unknown status" for other values). */
const char* pf8_strerror(pf8_status status);

/* PF8_ABI_VERSION of the loaded library. */
int pf8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PF8_H */
