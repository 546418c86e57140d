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

// Two independent 16-bit unsigned maxima in one instruction (v_pk_max_u16).
typedef unsigned short pf8_ushort2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  const pf8_ushort2 r = __builtin_elementwise_max(__builtin_bit_cast(pf8_ushort2, a), __builtin_bit_cast(pf8_ushort2, b));
  return __builtin_bit_cast(uint32_t, r);
}

// |bf16| bit patterns of the 8 values packed in v, reduced per half: the low 16 bits hold the
// largest of the four low halves, the high 16 bits the largest of the four high halves.
__device__ __forceinline__ uint32_t amax8_pk(uint4 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  return pk_max_u16(pk_max_u16(a, b), pk_max_u16(c, d));
}

// Largest |bf16| bit pattern among the 8 packed in v.
__device__ __forceinline__ uint32_t amax8_bits(uint4 v) {
  const uint32_t m = amax8_pk(v);
  return max(m & 0xFFFFu, m >> 16);
}

// From the per-half maxima of two rows (amax8_pk), both rows' maxima packed: row a in the low
// 16 bits, row b in the high 16 bits.
__device__ __forceinline__ uint32_t pair_amax(uint32_t pa, uint32_t pb) {
  return pk_max_u16(__builtin_amdgcn_perm(pb, pa, 0x05040100u), __builtin_amdgcn_perm(pb, pa, 0x07060302u));
}

// Two bf16 (one dword, low half first) divided by `scale` -> two OCP E4M3 codes, round to nearest
// even, packed into the low (HI = false) or high (HI = true) 16 bits of `old`: gfx950's
// v_cvt_scalef32_pk_fp8_bf16 in one instruction. With a power-of-two scale the division is exact,
// and the conversion was checked against the E4M3 definition on every finite bf16 value for
// scales 2^-127 .. 2^127.
typedef __bf16 pf8_bf16x2 __attribute__((ext_vector_type(2)));
typedef short pf8_short2 __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_bf16_scaled(uint32_t pair, float scale, uint32_t old) {
  const pf8_short2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(pf8_short2, old), __builtin_bit_cast(pf8_bf16x2, pair), scale, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 bf16 divided by `scale` (an exact power of two) -> 8 E4M3 codes.
__device__ __forceinline__ uint2 quant8_scaled(uint4 v, float scale) {
  const uint32_t lo = cvt2_bf16_scaled<true>(v.y, scale, cvt2_bf16_scaled<false>(v.x, scale, 0u));
  const uint32_t hi = cvt2_bf16_scaled<true>(v.w, scale, cvt2_bf16_scaled<false>(v.z, scale, 0u));
  return make_uint2(lo, hi);
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

// row16_max on two packed 16-bit values at once.
__device__ __forceinline__ uint32_t row16_max_pk(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  const int x = static_cast<int>(v);
  v = pk_max_u16(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false)));
  int y = static_cast<int>(v);
  v = pk_max_u16(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(y, y, 0x4E, 0xF, 0xF, false)));
  y = static_cast<int>(v);
  v = pk_max_u16(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(y, y, 0x141, 0xF, 0xF, false)));
  y = static_cast<int>(v);
  v = pk_max_u16(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(y, y, 0x140, 0xF, 0xF, false)));
  return v;
}

// Max over a full 64-lane wave (values are non-negative).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16)));
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32)));
  return v;
}

}  // namespace pf8
