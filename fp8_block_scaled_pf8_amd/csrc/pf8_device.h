// Device-side helpers shared by the libpf8 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf8 {

constexpr int kGroup = 128;  // block length along the reduction dimension

// Block exponent from the bit pattern of a block's absolute maximum (|bf16| bits, sign cleared).
// The scale 2^e is the smallest power of two with amax <= 448 * 2^e. Since 448 = 1.75 * 2^8,
// a normal amax = (1 + f/128) * 2^(E-127) needs e = E - 127 - 8, plus one when its significand
// exceeds 1.75 (f > 96). All-zero blocks use e = 0; e is clamped to >= -126 so 2^e is an fp32
// normal (bf16 subnormal maxima always land on the clamp).
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  const int ef = static_cast<int>(amax_bits >> 7);
  const int f = static_cast<int>(amax_bits & 0x7F);
  int e = ef - 135 + (f > 0x60 ? 1 : 0);
  e = e < -126 ? -126 : e;
  return amax_bits == 0 ? 0 : e;
}

// 2^e as an fp32 bit pattern, for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(static_cast<uint32_t>(127 + e) << 23); }

// Largest |bf16| bit pattern among the 8 packed in v.
__device__ __forceinline__ uint32_t amax8_bits(uint4 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  const uint32_t lo = max(max(a & 0xFFFFu, b & 0xFFFFu), max(c & 0xFFFFu, d & 0xFFFFu));
  const uint32_t hi = max(max(a >> 16, b >> 16), max(c >> 16, d >> 16));
  return max(lo, hi);
}

// bf16 (low / high half of a dword) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two OCP E4M3 codes (round to nearest even), packed into the low (hi=false) or
// high (hi=true) 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// 8 bf16 scaled by `inv` (an exact power of two) -> 8 E4M3 codes.
__device__ __forceinline__ uint2 quant8(uint4 v, float inv) {
  int lo = cvt2_e4m3<false>(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, 0);
  lo = cvt2_e4m3<true>(bf16_lo(v.y) * inv, bf16_hi(v.y) * inv, lo);
  int hi = cvt2_e4m3<false>(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, 0);
  hi = cvt2_e4m3<true>(bf16_lo(v.w) * inv, bf16_hi(v.w) * inv, hi);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// Max over the 16 lanes of a DPP row (a row of 16 lanes holds one 128-value group, 8 per lane).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  int x = static_cast<int>(v);
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return static_cast<uint32_t>(x);
}

// Max over a full 64-lane wave (values are non-negative).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16)));
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32)));
  return v;
}

}  // namespace pf8
