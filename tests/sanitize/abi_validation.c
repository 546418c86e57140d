/*
 * Host-side validation of every libpf8 entry point, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against the C ABI's host code and the stubs in host_stubs.cpp (no
 * device code, no HIP runtime: nothing is ever launched, and a call that passes validation returns
 * PF8_ENODEV). Each case states the status include/pf8.h promises. Extreme sizes (up to INT64_MAX)
 * check that the argument checks themselves are free of signed overflow.
 *
 * Exit status 0 and "ok <n> cases" when every call returns its expected status.
 */
#include <stdint.h>
#include <stdio.h>

#include "pf8.h"

static unsigned char buf[1 << 16] __attribute__((aligned(256)));
static int failures, cases;

static void expect(const char* what, int got, int want) {
  ++cases;
  if (got != want) {
    ++failures;
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
  }
}

#define CHECK(call, want) expect(#call, (call), (want))

int main(void) {
  void* p = buf;                      /* 16-byte aligned, never dereferenced by the library */
  void* q = buf + 4096;
  float* s = (float*)(buf + 8192);
  void* odd = buf + 8;                /* not 16-byte aligned */
  float* odd4 = (float*)(buf + 8194); /* not 4-byte aligned */
  const int64_t BIG = INT64_MAX;
  const int64_t BIG128 = INT64_MAX - INT64_MAX % 128; /* the largest multiple of 128 */

  /* ---- pf8_quant_act_1x128 ---- */
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_ENODEV);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_ROWS, q, 256, s, 512, 0), PF8_ENODEV);
  CHECK(pf8_quant_act_1x128(0, 256, 512, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, 0, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, q, 512, 0, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, 2, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, -1, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, 0x7FFFFFFF, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 0, 512, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, -128, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 500, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, 250, 512, 512, PF8_ALONG_ROWS, q, 256, s, 512, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, 256, 500, 512, PF8_ALONG_ROWS, q, 256, s, 512, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 511, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, q, 512, s, 255, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_1x128(odd, 256, 512, 512, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EALIGN);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, q, 512, odd4, 256, 0), PF8_EALIGN);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 516, PF8_ALONG_COLS, q, 512, s, 256, 0), PF8_EALIGN);
  CHECK(pf8_quant_act_1x128(p, 256, 512, 512, PF8_ALONG_COLS, q, 520, s, 256, 0), PF8_EALIGN);
  CHECK(pf8_quant_act_1x128(p, 256, 128 * 65536, 128 * 65536, PF8_ALONG_COLS, q, 128 * 65536, s, 256, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, BIG, 128, 128, PF8_ALONG_COLS, q, 128, s, BIG, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, 128, BIG128, BIG, PF8_ALONG_COLS, q, BIG, s, 128, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_1x128(p, BIG128, 128, BIG, PF8_ALONG_ROWS, q, BIG, s, BIG, 0), PF8_ESHAPE);

  /* ---- pf8_quant_act_dual ---- */
  CHECK(pf8_quant_act_dual(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, 0), PF8_ENODEV);
  CHECK(pf8_quant_act_dual(p, 256, 512, 512, q, 512, s, 256, 0, 256, s, 512, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_dual(p, 256, 500, 512, q, 512, s, 256, q, 256, s, 512, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_dual(p, 200, 512, 512, q, 512, s, 256, q, 256, s, 512, 0), PF8_ESHAPE);
  CHECK(pf8_quant_act_dual(p, 256, 512, 512, q, 512, s, 256, q, 255, s, 512, 0), PF8_EINVAL);
  CHECK(pf8_quant_act_dual(p, 256, 512, 512, q, 512, s, 256, odd, 256, s, 512, 0), PF8_EALIGN);
  CHECK(pf8_quant_act_dual(p, BIG128, BIG128, BIG, q, BIG, s, BIG, q, BIG, s, BIG, 0), PF8_ESHAPE);

  /* ---- pf8_quant_fwd ---- */
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, p, 384, 512, q, 512, q, 384, s, 4, 0),
        PF8_ENODEV);
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, p, 384, 512, q, 512, 0, 0, s, 4, 0),
        PF8_ENODEV);
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, 0, 384, 512, q, 512, q, 384, s, 4, 0),
        PF8_EINVAL);
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, p, 300, 512, q, 512, q, 384, s, 4, 0),
        PF8_ESHAPE);
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, p, 384, 512, q, 512, q, 383, s, 4, 0),
        PF8_EINVAL);
  CHECK(pf8_quant_fwd(p, 256, 512, 512, q, 512, s, 256, q, 256, s, 512, p, 384, 512, q, 512, odd, 384, s, 4, 0),
        PF8_EALIGN);
  CHECK(pf8_quant_fwd(p, BIG128, BIG128, BIG, q, BIG, s, BIG, q, BIG, s, BIG, p, BIG128, BIG, q, BIG, q, BIG, s, BIG,
                      0),
        PF8_ESHAPE);

  /* ---- pf8_quant_w_128x128 ---- */
  CHECK(pf8_quant_w_128x128(p, 384, 512, 512, q, 512, q, 384, s, 4, 0), PF8_ENODEV);
  CHECK(pf8_quant_w_128x128(p, 384, 512, 512, q, 512, 0, 0, s, 4, 0), PF8_ENODEV);
  CHECK(pf8_quant_w_128x128(0, 384, 512, 512, q, 512, q, 384, s, 4, 0), PF8_EINVAL);
  CHECK(pf8_quant_w_128x128(p, 384, 500, 512, q, 512, q, 384, s, 4, 0), PF8_ESHAPE);
  CHECK(pf8_quant_w_128x128(p, 384, 512, 512, q, 512, q, 384, s, 3, 0), PF8_EINVAL);
  CHECK(pf8_quant_w_128x128(p, 384, 512, 512, q, 512, odd, 384, s, 4, 0), PF8_EALIGN);
  CHECK(pf8_quant_w_128x128(p, 384, 512, 512, q, 512, q, 392, s, 4, 0), PF8_EALIGN);
  CHECK(pf8_quant_w_128x128(p, BIG128, BIG128, BIG, q, BIG, q, BIG, s, BIG, 0), PF8_ESHAPE);

  /* ---- pf8_block_gemm, pf8_block_gemm_variant ---- */
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_ENODEV);
  CHECK(pf8_block_gemm(PF8_WGRAD, 300, 200, 384, p, 384, s, 300, q, 384, s, 1, 200, p, 200, 0), PF8_ENODEV);
  CHECK(pf8_block_gemm(3, 300, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(-1, 300, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm_variant(3, PF8_FPROP, 300, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm_variant(PF8_GEMM_PROMOTE, PF8_DGRAD, 300, 200, 384, p, 384, s, 300, q, 384, s, 1, 3, p, 200, 0),
        PF8_ENODEV);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, 0, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(PF8_FPROP, 0, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 300, p, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_ESHAPE);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 383, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, s, 299, q, 384, s, 3, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, s, 300, q, 384, s, 0, 1, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 392, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EALIGN);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, s, 300, q, 384, s, 3, 1, p, 204, 0), PF8_EALIGN);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, odd, 384, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EALIGN);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 384, odd4, 300, q, 384, s, 3, 1, p, 200, 0), PF8_EALIGN);
  CHECK(pf8_block_gemm(PF8_FPROP, 300, 200, 384, p, 8388608, s, 300, q, 384, s, 3, 1, p, 200, 0), PF8_ESHAPE);
  CHECK(pf8_block_gemm(PF8_FPROP, BIG, BIG, BIG128, p, BIG, s, BIG, q, BIG, s, BIG, BIG, p, BIG, 0), PF8_ESHAPE);
  CHECK(pf8_block_gemm(PF8_FPROP, BIG, BIG, 128, p, 128, s, BIG, q, 128, s, 1, 1, p, BIG, 0), PF8_ESHAPE);

  /* ---- pf8_block_gemm_f32 ---- */
  CHECK(pf8_block_gemm_f32(PF8_WGRAD, 300, 200, 384, p, 384, s, 300, q, 384, s, 1, 200, (float*)p, 200, 1, 0),
        PF8_ENODEV);
  CHECK(pf8_block_gemm_f32(PF8_WGRAD, 300, 200, 384, p, 384, s, 300, q, 384, s, 1, 200, (float*)p, 200, 2, 0),
        PF8_EINVAL);
  CHECK(pf8_block_gemm_f32(PF8_WGRAD, 300, 200, 384, p, 384, s, 300, q, 384, s, 1, 200, (float*)p, 202, 0, 0),
        PF8_EALIGN);
  CHECK(pf8_block_gemm_f32(PF8_FPROP, BIG, BIG, 128, p, 128, s, BIG, q, 128, s, 1, 1, (float*)p, BIG, 0, 0),
        PF8_ESHAPE);

  /* ---- pf8_gemm_bf16 ---- */
  CHECK(pf8_gemm_bf16(300, 200, 384, p, 384, q, 384, p, 200, 0), PF8_ENODEV);
  CHECK(pf8_gemm_bf16(300, 200, 384, 0, 384, q, 384, p, 200, 0), PF8_EINVAL);
  CHECK(pf8_gemm_bf16(300, 200, 384, p, 388, q, 384, p, 200, 0), PF8_EALIGN);
  CHECK(pf8_gemm_bf16(300, 200, 384, p, 4194304, q, 384, p, 200, 0), PF8_ESHAPE);
  CHECK(pf8_gemm_bf16(300, 200, BIG128, p, BIG, q, BIG, p, 200, 0), PF8_ESHAPE);
  CHECK(pf8_gemm_bf16(BIG, BIG, 128, p, 128, q, 128, p, BIG, 0), PF8_ESHAPE);

  /* ---- strings and version ---- */
  for (int st = -2; st < 8; ++st) {
    const char* m = pf8_strerror(st);
    ++cases;
    if (m == 0 || m[0] == 0) {
      ++failures;
      printf("FAIL pf8_strerror(%d)\n", st);
    }
  }
  CHECK(pf8_abi_version(), PF8_ABI_VERSION);

  if (failures) {
    printf("%d of %d cases failed\n", failures, cases);
    return 1;
  }
  printf("ok %d cases\n", cases);
  return 0;
}
