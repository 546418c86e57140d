// C ABI of libpf8 (declared in include/pf8.h): host-side validation and dispatch.
//
// Every argument is checked before anything is enqueued; the checks need no GPU, so the library
// loads and validates on a machine without one (and then reports PF8_ENODEV for valid calls).
#include <stdint.h>

#include "../../include/pf8.h"
#include "pf8_launch.h"

namespace {

constexpr int64_t kGroup = 128;
constexpr int64_t kMaxTilePitch = ((int64_t{1} << 31) - 1) / 256;  // 256 rows x pitch must fit a signed 32-bit offset

// Every dimension, leading dimension and scale stride is at most 2^31 - 1 (PF8_ESHAPE otherwise):
// no array that large fits a GPU's memory, and the bound keeps every size product and pitch in
// bytes below 2^63, so the checks below cannot overflow.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
template <typename... T>
bool any_too_big(T... v) {
  return ((v > kMaxDim) || ...);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int device_status() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return PF8_ENODEV;
  }
  return PF8_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PF8_OK : PF8_ELAUNCH; }

}  // namespace

extern "C" {

int pf8_abi_version(void) { return PF8_ABI_VERSION; }

const char* pf8_strerror(pf8_status status) {
  switch (status) {
    case PF8_OK: return "ok";
    case PF8_EINVAL: return "invalid argument (null pointer, unknown enum, non-positive dimension or leading dimension too small)";
    case PF8_ESHAPE: return "unsupported shape (a grouped or tiled dimension is not a multiple of 128, col-mode cols not a multiple of 8, or a pitch too large)";
    case PF8_EALIGN: return "misaligned buffer (base not 16-byte aligned or row pitch not a multiple of 16 bytes)";
    case PF8_ENODEV: return "no HIP device available";
    case PF8_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

pf8_status pf8_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx, pf8_group_axis axis, void* q, int64_t ldq,
                        float* dscale, int64_t ld_s, void* hip_stream) {
  if (x == nullptr || q == nullptr || dscale == nullptr) return PF8_EINVAL;
  if (axis != PF8_ALONG_COLS && axis != PF8_ALONG_ROWS) return PF8_EINVAL;
  if (rows <= 0 || cols <= 0) return PF8_EINVAL;
  if (any_too_big(rows, cols, ldx, ldq, ld_s)) return PF8_ESHAPE;
  if (ldx < cols) return PF8_EINVAL;
  if (axis == PF8_ALONG_COLS) {
    if (cols % kGroup != 0) return PF8_ESHAPE;
    if (ldq < cols || ld_s < rows) return PF8_EINVAL;
  } else {
    if (rows % kGroup != 0 || cols % 8 != 0) return PF8_ESHAPE;
    if (ldq < rows || ld_s < cols) return PF8_EINVAL;
  }
  if (!aligned16(x) || !aligned16(q) || !aligned4(dscale) || (ldx * 2) % 16 != 0 || ldq % 16 != 0) return PF8_EALIGN;
  // one grid row per 128-group of a row (row mode) or per 128-row band (col mode)
  if ((axis == PF8_ALONG_COLS ? cols : rows) / kGroup > 65535) return PF8_ESHAPE;
  if (int s = device_status(); s != PF8_OK) return s;
  auto stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = axis == PF8_ALONG_COLS ? pf8::launch_quant_rows(x, rows, cols, ldx, q, ldq, dscale, ld_s, stream)
                                              : pf8::launch_quant_cols(x, rows, cols, ldx, q, ldq, dscale, ld_s, stream);
  return launch_status(e);
}

pf8_status pf8_quant_act_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, int64_t ldq_row,
                       float* dscale_row, int64_t ld_sr, void* q_col, int64_t ldq_col, float* dscale_col, int64_t ld_sc,
                       void* hip_stream) {
  if (x == nullptr || q_row == nullptr || dscale_row == nullptr || q_col == nullptr || dscale_col == nullptr)
    return PF8_EINVAL;
  if (rows <= 0 || cols <= 0) return PF8_EINVAL;
  if (any_too_big(rows, cols, ldx, ldq_row, ld_sr, ldq_col, ld_sc)) return PF8_ESHAPE;
  if (rows % kGroup != 0 || cols % kGroup != 0) return PF8_ESHAPE;
  if (ldx < cols || ldq_row < cols || ld_sr < rows || ldq_col < rows || ld_sc < cols) return PF8_EINVAL;
  if (!aligned16(x) || !aligned16(q_row) || !aligned16(q_col) || !aligned4(dscale_row) || !aligned4(dscale_col))
    return PF8_EALIGN;
  if ((ldx * 2) % 16 != 0 || ldq_row % 16 != 0 || ldq_col % 16 != 0) return PF8_EALIGN;
  if (rows / kGroup > 65535 || cols / kGroup > (int64_t{1} << 31) - 1) return PF8_ESHAPE;  // grid (cols/128, rows/128)
  if (int s = device_status(); s != PF8_OK) return s;
  return launch_status(pf8::launch_quant_dual(x, rows, cols, ldx, q_row, ldq_row, dscale_row, ld_sr, q_col, ldq_col,
                                              dscale_col, ld_sc, static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_quant_fwd(const void* x, int64_t m, int64_t k, int64_t ldx, void* qx, int64_t ldqx, float* sx, int64_t ld_sx,
                  void* qxt, int64_t ldqxt, float* sxt, int64_t ld_sxt, const void* w, int64_t n, int64_t ldw, void* qw,
                  int64_t ldqw, void* qwt, int64_t ldqwt, float* sw, int64_t ld_sw, void* hip_stream) {
  if (x == nullptr || qx == nullptr || sx == nullptr || qxt == nullptr || sxt == nullptr || w == nullptr ||
      qw == nullptr || sw == nullptr)
    return PF8_EINVAL;
  if (m <= 0 || n <= 0 || k <= 0) return PF8_EINVAL;
  if (any_too_big(m, n, k, ldx, ldqx, ld_sx, ldqxt, ld_sxt, ldw, ldqw, ld_sw, qwt != nullptr ? ldqwt : 0))
    return PF8_ESHAPE;
  if (m % kGroup != 0 || n % kGroup != 0 || k % kGroup != 0) return PF8_ESHAPE;
  if (ldx < k || ldqx < k || ld_sx < m || ldqxt < m || ld_sxt < k) return PF8_EINVAL;
  if (ldw < k || ldqw < k || ld_sw < k / kGroup || (qwt != nullptr && ldqwt < n)) return PF8_EINVAL;
  if (!aligned16(x) || !aligned16(qx) || !aligned16(qxt) || !aligned4(sx) || !aligned4(sxt)) return PF8_EALIGN;
  if (!aligned16(w) || !aligned16(qw) || !aligned4(sw) || (qwt != nullptr && !aligned16(qwt))) return PF8_EALIGN;
  if ((ldx * 2) % 16 != 0 || ldqx % 16 != 0 || ldqxt % 16 != 0 || (ldw * 2) % 16 != 0 || ldqw % 16 != 0 ||
      (qwt != nullptr && ldqwt % 16 != 0))
    return PF8_EALIGN;
  if ((m / kGroup + n / kGroup) * (k / kGroup) > (int64_t{1} << 31) - 1) return PF8_ESHAPE;  // one workgroup per tile
  if (int s = device_status(); s != PF8_OK) return s;
  return launch_status(pf8::launch_quant_fwd(x, m, k, ldx, qx, ldqx, sx, ld_sx, qxt, ldqxt, sxt, ld_sxt, w, n, ldw, qw,
                                             ldqw, qwt, ldqwt, sw, ld_sw, static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_quant_w_128x128(const void* w, int64_t n, int64_t k, int64_t ldw, void* q, int64_t ldq, void* qt, int64_t ldqt,
                        float* dscale, int64_t ld_s, void* hip_stream) {
  if (w == nullptr || q == nullptr || dscale == nullptr) return PF8_EINVAL;
  if (n <= 0 || k <= 0) return PF8_EINVAL;
  if (any_too_big(n, k, ldw, ldq, ld_s, qt != nullptr ? ldqt : 0)) return PF8_ESHAPE;
  if (n % kGroup != 0 || k % kGroup != 0) return PF8_ESHAPE;
  if (ldw < k || ldq < k || ld_s < k / kGroup || (qt != nullptr && ldqt < n)) return PF8_EINVAL;
  if (!aligned16(w) || !aligned16(q) || !aligned4(dscale) || (ldw * 2) % 16 != 0 || ldq % 16 != 0) return PF8_EALIGN;
  if (qt != nullptr && (!aligned16(qt) || ldqt % 16 != 0)) return PF8_EALIGN;
  if (n / kGroup > 65535) return PF8_ESHAPE;  // one grid row per 128-row tile band
  if (int s = device_status(); s != PF8_OK) return s;
  return launch_status(pf8::launch_quant_w(w, n, k, ldw, q, ldq, qt, ldqt, dscale, ld_s,
                                           static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_block_gemm_variant(int variant, pf8_layout layout, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                           const float* a_dscale, int64_t ld_as, const void* b, int64_t ldb, const float* b_dscale,
                           int64_t sb_n, int64_t sb_k, void* d, int64_t ldd, void* hip_stream) {
  if (variant != PF8_GEMM_AUTO && variant != PF8_GEMM_MX_SCALED && variant != PF8_GEMM_PROMOTE) return PF8_EINVAL;
  if (layout != PF8_FPROP && layout != PF8_DGRAD && layout != PF8_WGRAD) return PF8_EINVAL;
  if (a == nullptr || b == nullptr || d == nullptr || a_dscale == nullptr || b_dscale == nullptr) return PF8_EINVAL;
  if (m <= 0 || n <= 0 || k <= 0) return PF8_EINVAL;
  if (any_too_big(m, n, k, lda, ldb, ldd, ld_as, sb_n, sb_k)) return PF8_ESHAPE;
  if (k % kGroup != 0) return PF8_ESHAPE;
  if (lda < k || ldb < k || ldd < n || ld_as < m || sb_n < 1 || sb_k < 1) return PF8_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d) || !aligned4(a_dscale) || !aligned4(b_dscale)) return PF8_EALIGN;
  if (lda % 16 != 0 || ldb % 16 != 0 || (ldd * 2) % 16 != 0) return PF8_EALIGN;
  if (lda > kMaxTilePitch || ldb > kMaxTilePitch) return PF8_ESHAPE;
  if ((m + 127) / 128 * ((n + 127) / 128) > (int64_t{1} << 31) - 1) return PF8_ESHAPE;
  if (int s = device_status(); s != PF8_OK) return s;
  pf8::GemmArgs args{m, n, k, static_cast<const uint8_t*>(a), lda, a_dscale, ld_as, static_cast<const uint8_t*>(b),
                     ldb, b_dscale, sb_n, sb_k, static_cast<uint16_t*>(d), ldd, nullptr, 0};
  const bool mx = variant != PF8_GEMM_PROMOTE;
  return launch_status(pf8::launch_gemm(args, layout == PF8_WGRAD, mx, static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_block_gemm_f32(pf8_layout layout, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const float* a_dscale,
                       int64_t ld_as, const void* b, int64_t ldb, const float* b_dscale, int64_t sb_n, int64_t sb_k,
                       float* d, int64_t ldd, int accumulate, void* hip_stream) {
  if (layout != PF8_FPROP && layout != PF8_DGRAD && layout != PF8_WGRAD) return PF8_EINVAL;
  if (accumulate != 0 && accumulate != 1) return PF8_EINVAL;
  if (a == nullptr || b == nullptr || d == nullptr || a_dscale == nullptr || b_dscale == nullptr) return PF8_EINVAL;
  if (m <= 0 || n <= 0 || k <= 0) return PF8_EINVAL;
  if (any_too_big(m, n, k, lda, ldb, ldd, ld_as, sb_n, sb_k)) return PF8_ESHAPE;
  if (k % kGroup != 0) return PF8_ESHAPE;
  if (lda < k || ldb < k || ldd < n || ld_as < m || sb_n < 1 || sb_k < 1) return PF8_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d) || !aligned4(a_dscale) || !aligned4(b_dscale)) return PF8_EALIGN;
  if (lda % 16 != 0 || ldb % 16 != 0 || (ldd * 4) % 16 != 0) return PF8_EALIGN;
  if (lda > kMaxTilePitch || ldb > kMaxTilePitch) return PF8_ESHAPE;
  if ((m + 127) / 128 * ((n + 127) / 128) > (int64_t{1} << 31) - 1) return PF8_ESHAPE;
  if (int s = device_status(); s != PF8_OK) return s;
  pf8::GemmArgs args{m, n, k, static_cast<const uint8_t*>(a), lda, a_dscale, ld_as, static_cast<const uint8_t*>(b),
                     ldb, b_dscale, sb_n, sb_k, nullptr, ldd, d, accumulate};
  return launch_status(pf8::launch_gemm(args, layout == PF8_WGRAD, true, static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_gemm_bf16(int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const void* b, int64_t ldb, void* d,
                  int64_t ldd, void* hip_stream) {
  if (a == nullptr || b == nullptr || d == nullptr) return PF8_EINVAL;
  if (m <= 0 || n <= 0 || k <= 0) return PF8_EINVAL;
  if (any_too_big(m, n, k, lda, ldb, ldd)) return PF8_ESHAPE;
  if (k % kGroup != 0) return PF8_ESHAPE;
  if (lda < k || ldb < k || ldd < n) return PF8_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(d)) return PF8_EALIGN;
  if ((lda * 2) % 16 != 0 || (ldb * 2) % 16 != 0 || (ldd * 2) % 16 != 0) return PF8_EALIGN;
  if (lda * 2 > kMaxTilePitch || ldb * 2 > kMaxTilePitch) return PF8_ESHAPE;
  if ((m + 127) / 128 * ((n + 127) / 128) > (int64_t{1} << 31) - 1) return PF8_ESHAPE;
  if (int s = device_status(); s != PF8_OK) return s;
  // the kernel streams bytes: K and the pitches in bytes, no scales
  pf8::GemmArgs args{m, n, 2 * k, static_cast<const uint8_t*>(a), 2 * lda, nullptr, 0, static_cast<const uint8_t*>(b),
                     2 * ldb, nullptr, 0, 0, static_cast<uint16_t*>(d), ldd, nullptr, 0};
  return launch_status(pf8::launch_gemm_bf16(args, static_cast<hipStream_t>(hip_stream)));
}

pf8_status pf8_block_gemm(pf8_layout layout, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const float* a_dscale,
                   int64_t ld_as, const void* b, int64_t ldb, const float* b_dscale, int64_t sb_n, int64_t sb_k,
                   void* d, int64_t ldd, void* hip_stream) {
  return pf8_block_gemm_variant(PF8_GEMM_AUTO, layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k,
                                d, ldd, hip_stream);
}

}  // extern "C"
