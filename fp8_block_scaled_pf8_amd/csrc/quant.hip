// Online power-of-two E4M3 quantisers for gfx950.
//
// Method [Puro-2B report; paper.rainbus.top summary, section "FP8 块级混合精度训练" and
// 方法步骤详情 step (3); ta-paperlens explainer, 打ち手2 (report §3.2)]: one power-of-two scale per
// 128 values along the reduction dimension for activations/gradients, per 128x128 tile for
// weights, each computed from its own block when the tensor is quantised.
//
// All kernels are HBM-bound streams (2 B read + ~1 B written per element and grouping): one read
// of the input, block maxima reduced in registers / across lanes, then gfx950's scaled conversion
// (v_cvt_scalef32_pk_fp8_bf16: two bf16 divided by the power-of-two scale and rounded to E4M3,
// nearest even, in one instruction) straight from the bf16 words.
#include "pf8_device.h"
#include "pf8_launch.h"

namespace pf8 {

typedef unsigned int pf8_u32x4 __attribute__((ext_vector_type(4)));  // for non-temporal 16-byte loads

// ---------------------------------------------------------------------------------------------
// Row mode: a group is 128 consecutive elements of a row (16 lanes x 8 bf16).
// Grid: x over row blocks of 16 * kRowUnroll rows, y over the cols / 128 groups of a row.
// Lane slice s (16 lanes) of the workgroup handles rows r0 + s + 16 * u, u < kRowUnroll.
constexpr int kRowUnroll = 4;
constexpr int kRowsPerWG = 16 * kRowUnroll;

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ dscale, int64_t ld_s) {
  const int lane16 = threadIdx.x & 15;
  const int slice = threadIdx.x >> 4;
  const int64_t g = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + slice;
  uint4 v[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int64_t r = r0 + 16 * u;
    v[u] = make_uint4(0, 0, 0, 0);
    // non-temporal: the input is read once here (the layer step with one pass per orientation,
    // interleaved: 703.6 -> 688.9 us, mostly in the GEMMs that follow)
    if (r < rows)
      v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                           reinterpret_cast<const pf8_u32x4*>(x + r * ldx + g * kGroup + lane16 * 8)));
  }
  static_assert(kRowUnroll % 2 == 0, "rows are reduced in pairs");
#pragma unroll
  for (int k = 0; k < kRowUnroll / 2; ++k) {
    // every lane of the 16-lane row takes part in the reduction (rows past the end hold zeros);
    // two rows' maxima travel through the DPP reduction packed in one register
    const uint32_t amax2 = row16_max_pk(pair_amax(amax8_pk(v[2 * k]), amax8_pk(v[2 * k + 1])));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int u = 2 * k + hh;
      const int64_t r = r0 + 16 * u;
      const float scale = pow2f(block_exponent(hh ? amax2 >> 16 : amax2 & 0xFFFFu));
      const uint2 codes = quant8_scaled(v[u], scale);
      if (r < rows) {
        *reinterpret_cast<uint2*>(q + r * ldq + g * kGroup + lane16 * 8) = codes;
        if (lane16 == 0) dscale[g * ld_s + r] = scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Col mode: a group is 128 consecutive rows of one column; codes are written transposed
// (q[c][r], rows contiguous). A workgroup quantises a 128-row x 64-column tile:
//   thread t holds columns 8*(t%8) .. +7 of rows 4*(t/8) .. +3 (four 16-byte loads),
//   column maxima are reduced over lanes (xor 8, 16, 32) and then over the 4 waves in LDS,
//   codes go to an LDS tile [64 cols][128 rows] bytes and leave as 128-byte rows.
// LDS 16-byte chunk ch of tile row c is stored at chunk ch ^ ((c >> 3) & 7) to spread banks.
constexpr int kColTile = 64;

__global__ __launch_bounds__(256) void quant_cols_kernel(const uint16_t* __restrict__ x, int64_t cols, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ dscale, int64_t ld_s) {
  __shared__ uint32_t red[4][kColTile];
  __shared__ __align__(16) uint8_t tile[kColTile * kGroup];
  const int t = threadIdx.x;
  const int cc = t & 7;      // column chunk: columns 8*cc .. 8*cc+7 of the tile
  const int rq = t >> 3;     // row quad: rows 4*rq .. 4*rq+3 of the group
  const int wave = t >> 6;
  const int64_t g = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kColTile;
  const int64_t col = c0 + 8 * cc;
  const bool col_ok = col < cols;  // cols % 8 == 0, so a chunk is all in or all out
  uint4 v[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    v[p] = make_uint4(0, 0, 0, 0);
    if (col_ok)  // non-temporal, as in row mode
      v[p] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                           reinterpret_cast<const pf8_u32x4*>(x + (g * kGroup + 4 * rq + p) * ldx + col)));
  }
  // per-column max of |x| over this thread's 4 rows; column j of the chunk lives in half (j&1) of word j/2
  uint32_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      m[2 * h] = max(m[2 * h], w[h] & 0x7FFFu);
      m[2 * h + 1] = max(m[2 * h + 1], (w[h] >> 16) & 0x7FFFu);
    }
  }
  // reduce over the 8 row quads of this wave (lanes differing in bits 3..5 share a column chunk)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t a = m[j];
    a = max(a, static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), 8)));
    a = max(a, static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), 16)));
    a = max(a, static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), 32)));
    m[j] = a;
  }
  if ((t & 63) < 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][8 * cc + j] = m[j];
  }
  __syncthreads();
  float scale[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cc + j;
    const uint32_t a = max(max(red[0][c], red[1][c]), max(red[2][c], red[3][c]));
    scale[j] = pow2f(block_exponent(a));
    if (rq == 0 && col_ok) dscale[g * ld_s + c0 + c] = scale[j];
  }
  // quantise: for column j, the 4 codes of rows 4rq..4rq+3 form one little-endian dword; the
  // column's values of two rows are paired into one dword (v_perm) and converted together
  uint32_t colword[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int h = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each row's word
    const uint32_t w0 = h == 0 ? v[0].x : h == 1 ? v[0].y : h == 2 ? v[0].z : v[0].w;
    const uint32_t w1 = h == 0 ? v[1].x : h == 1 ? v[1].y : h == 2 ? v[1].z : v[1].w;
    const uint32_t w2 = h == 0 ? v[2].x : h == 1 ? v[2].y : h == 2 ? v[2].z : v[2].w;
    const uint32_t w3 = h == 0 ? v[3].x : h == 1 ? v[3].y : h == 2 ? v[3].z : v[3].w;
    const uint32_t p01 = __builtin_amdgcn_perm(w1, w0, sel), p23 = __builtin_amdgcn_perm(w3, w2, sel);
    colword[j] = cvt2_bf16_scaled<true>(p23, scale[j], cvt2_bf16_scaled<false>(p01, scale[j], 0u));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cc + j;
    const int ch = (rq >> 2) ^ ((c >> 3) & 7);
    *reinterpret_cast<uint32_t*>(tile + c * kGroup + ch * 16 + (rq & 3) * 4) = colword[j];
  }
  __syncthreads();
  // write out: 64 rows of 128 bytes; thread t handles chunk (t & 7) of tile rows (t >> 3) and (t >> 3) + 32
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = (t >> 3) + 32 * h;
    const int ch = t & 7;
    const uint4 val = *reinterpret_cast<const uint4*>(tile + c * kGroup + ((ch ^ ((c >> 3) & 7)) * 16));
    if (c0 + c < cols) *reinterpret_cast<uint4*>(q + (c0 + c) * ldq + g * kGroup + ch * 16) = val;
  }
}

// ---------------------------------------------------------------------------------------------
// Weight tiles: one workgroup per 128x128 tile.
//   thread t holds the 8x8 block rows 8*(t/16) .. +7, columns 8*(t%16) .. +7 (eight 16-byte loads);
//   the tile maximum is reduced over the wave and then over the 4 waves in LDS;
//   codes go straight to q[n][k] (8 bytes per row per thread) and, when qt is requested,
//   through an LDS tile [128 k][128 n] bytes to qt[k][n].
// (red: 4 words of LDS, tile: kGroup * kGroup bytes of LDS, both owned by the workgroup)
__device__ __forceinline__ void quant_w_tile(const uint16_t* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q,
                                             int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt,
                                             float* __restrict__ dscale, int64_t ld_s, int64_t tn, int64_t tk,
                                             uint32_t* red, uint8_t* tile) {
  const int t = threadIdx.x;
  const int rb = t >> 4;  // row block: rows 8*rb .. 8*rb+7
  const int cb = t & 15;  // col block: cols 8*cb .. 8*cb+7
  const int64_t row0 = tn * kGroup + 8 * rb;
  const int64_t col0 = tk * kGroup + 8 * cb;
  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) v[p] = *reinterpret_cast<const uint4*>(w + (row0 + p) * ldw + col0);
  uint32_t a = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) a = max(a, amax8_bits(v[p]));
  a = wave_max(a);
  if ((t & 63) == 0) red[t >> 6] = a;
  __syncthreads();
  a = max(max(red[0], red[1]), max(red[2], red[3]));
  const float scale = pow2f(block_exponent(a));
  if (t == 0) dscale[tn * ld_s + tk] = scale;
  uint2 codes[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    codes[p] = quant8_scaled(v[p], scale);
    *reinterpret_cast<uint2*>(q + (row0 + p) * ldq + col0) = codes[p];
  }
  if (qt == nullptr) return;  // uniform over the workgroup
  // 8x8 byte transpose in registers: column j's 8 bytes (rows p = 0..7) form one 64-bit word
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t word = (j < 4) ? codes[p].x : codes[p].y;
      const uint32_t byte = (word >> (8 * (j & 3))) & 0xFFu;
      if (p < 4) lo |= byte << (8 * p);
      else hi |= byte << (8 * (p - 4));
    }
    const int c = 8 * cb + j;                 // tile row of qt (a column of w)
    const int ch = (rb >> 1) ^ ((c >> 3) & 7);  // 16-byte chunk holding rows 8*rb .. 8*rb+7
    *reinterpret_cast<uint2*>(tile + c * kGroup + ch * 16 + (rb & 1) * 8) = make_uint2(lo, hi);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int c = (t >> 3) + 32 * h;
    const int ch = t & 7;
    const uint4 val = *reinterpret_cast<const uint4*>(tile + c * kGroup + ((ch ^ ((c >> 3) & 7)) * 16));
    *reinterpret_cast<uint4*>(qt + (tk * kGroup + c) * ldqt + tn * kGroup + ch * 16) = val;
  }
}

__global__ __launch_bounds__(256) void quant_w_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                      uint8_t* __restrict__ q, int64_t ldq,
                                                      uint8_t* __restrict__ qt, int64_t ldqt,
                                                      float* __restrict__ dscale, int64_t ld_s) {
  __shared__ uint32_t red[4];
  __shared__ __align__(16) uint8_t tile[kGroup * kGroup];
  quant_w_tile(w, ldw, q, ldq, qt, ldqt, dscale, ld_s, blockIdx.y, blockIdx.x, red, tile);
}

// ---------------------------------------------------------------------------------------------
// Both orientations from one read: a workgroup takes a 128 x 128 tile, which is 128 row groups
// (one per row, along the columns) and 128 column groups (one per column, along the rows).
//   thread t holds rows 8*(t/16) .. +7, columns 8*(t%16) .. +7 (eight 16-byte loads);
//   row mode: a row's maximum is reduced over its 16 lanes (one DPP row), codes go straight out;
//   col mode: per-column maxima over the thread's 8 rows (packed 16-bit max), then over the wave
//   (xor 16, 32) and the 4 waves in LDS; for column j the thread's 8 codes (rows 8*(t/16) ..)
//   form one 64-bit word, written to an LDS tile [128 cols][128 rows] and sent out as 128-byte
//   rows of the transposed code matrix.
// LDS tile: rows c, c+1 (c even) share 256 bytes = all 64 banks; 8-byte slot s of row c sits at
// slot (s | (c & 1) << 4) ^ (((c >> 3) & 7) << 2) of the pair, so a 16-lane read of two rows'
// 16-byte chunks touches every bank once.
__device__ __forceinline__ int dual_slot(int c, int s) {
  return (c >> 1) * 256 + 8 * ((s | ((c & 1) << 4)) ^ (((c >> 3) & 7) << 2));
}

// (red: [wave][column chunk][packed column pair] words of LDS, tile: kGroup * kGroup bytes of LDS;
// gc = column group (row mode), gr = row group (col mode))
// The BF16 input is read with non-temporal loads, so a tensor that is read once does not displace
// what the following GEMMs read from the caches. The standalone dual quantiser on dY of the
// gate+up layer step: step 652.0 -> 631.6 us, the weight gradient 191.7 -> 177.9 us. The forward
// quantiser's X tiles, interleaved A/B over 15 rounds: dgrad 3.1 us and wgrad 2.2 us faster, the
// step 5.5 us (the likely reason: more of the weight codes and of X's transposed codes, which
// those GEMMs read, stay in the caches). The weight tiles keep cached loads: non-temporal ones
// there slowed fprop.
__device__ __forceinline__ void quant_dual_tile(const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ qr,
                                                int64_t ldqr, float* __restrict__ sr, int64_t ld_sr,
                                                uint8_t* __restrict__ qc, int64_t ldqc, float* __restrict__ sc,
                                                int64_t ld_sc, int64_t gc, int64_t gr, uint32_t (*red)[16][4],
                                                uint8_t* tile) {
  const int t = threadIdx.x;
  const int rb = t >> 4;  // rows 8*rb .. 8*rb+7 of the tile
  const int cc = t & 15;  // cols 8*cc .. 8*cc+7 of the tile
  const int wave = t >> 6;
  const int64_t r0 = gr * kGroup, c0 = gc * kGroup;
  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint16_t* src = x + (r0 + 8 * rb + p) * ldx + c0 + 8 * cc;
    v[p] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const pf8_u32x4*>(src)));
  }

  // ---- row mode: 8 rows, one 128-value group each ----
  // (row maxima two at a time: packed 16-bit pairs through the DPP reduction)
  float my_row_scale = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t rm = row16_max_pk(pair_amax(amax8_pk(v[2 * k]), amax8_pk(v[2 * k + 1])));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int p = 2 * k + hh;
      const float scale = pow2f(block_exponent(hh ? rm >> 16 : rm & 0xFFFFu));
      *reinterpret_cast<uint2*>(qr + (r0 + 8 * rb + p) * ldqr + c0 + 8 * cc) = quant8_scaled(v[p], scale);
      if (cc == p) my_row_scale = scale;
    }
  }
  if (cc < 8) sr[gc * ld_sr + r0 + 8 * rb + cc] = my_row_scale;

  // ---- col mode: per-column maxima, packed as column pairs (2h, 2h+1) in word h ----
  uint32_t m[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) m[h] = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) m[h] = pk_max_u16(m[h], w[h] & 0x7FFF7FFFu);
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m[h] = pk_max_u16(m[h], static_cast<uint32_t>(__shfl_xor(static_cast<int>(m[h]), 16)));
    m[h] = pk_max_u16(m[h], static_cast<uint32_t>(__shfl_xor(static_cast<int>(m[h]), 32)));
  }
  if ((t & 63) < 16) *reinterpret_cast<uint4*>(&red[wave][cc][0]) = make_uint4(m[0], m[1], m[2], m[3]);
  __syncthreads();
  float scale[8];
  {
    uint4 a = *reinterpret_cast<const uint4*>(&red[0][cc][0]);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const uint4 b = *reinterpret_cast<const uint4*>(&red[w][cc][0]);
      a = make_uint4(pk_max_u16(a.x, b.x), pk_max_u16(a.y, b.y), pk_max_u16(a.z, b.z), pk_max_u16(a.w, b.w));
    }
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    float my_col_scale = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      scale[j] = pow2f(block_exponent((aw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
      if (rb == j) my_col_scale = scale[j];
    }
    // thread (rb < 8, cc) writes the scale of column 8*cc + rb
    if (rb < 8) sc[gr * ld_sc + c0 + 8 * cc + rb] = my_col_scale;
  }
  // codes of column j for rows 8*rb .. 8*rb+7: one little-endian 64-bit word; the column's
  // values of rows p, p+1 are paired into one dword (v_perm) and converted together
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int h = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each row's word
    uint32_t w[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) w[p] = h == 0 ? v[p].x : h == 1 ? v[p].y : h == 2 ? v[p].z : v[p].w;
    const uint32_t lo = cvt2_bf16_scaled<true>(__builtin_amdgcn_perm(w[3], w[2], sel), scale[j],
                                               cvt2_bf16_scaled<false>(__builtin_amdgcn_perm(w[1], w[0], sel), scale[j], 0u));
    const uint32_t hi = cvt2_bf16_scaled<true>(__builtin_amdgcn_perm(w[7], w[6], sel), scale[j],
                                               cvt2_bf16_scaled<false>(__builtin_amdgcn_perm(w[5], w[4], sel), scale[j], 0u));
    *reinterpret_cast<uint2*>(tile + dual_slot(8 * cc + j, rb)) = make_uint2(lo, hi);
  }
  __syncthreads();
  // 128 transposed rows of 128 bytes: thread t sends chunk (t & 7) of rows (t >> 3) + 32 * i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (t >> 3) + 32 * i;
    const int k = t & 7;
    const uint4 val = *reinterpret_cast<const uint4*>(tile + dual_slot(c, 2 * k));
    *reinterpret_cast<uint4*>(qc + (c0 + c) * ldqc + r0 + 16 * k) = val;
  }
}

__global__ __launch_bounds__(256) void quant_dual_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                         uint8_t* __restrict__ qr, int64_t ldqr,
                                                         float* __restrict__ sr, int64_t ld_sr,
                                                         uint8_t* __restrict__ qc, int64_t ldqc,
                                                         float* __restrict__ sc, int64_t ld_sc) {
  __shared__ __align__(16) uint32_t red[4][16][4];
  __shared__ __align__(16) uint8_t tile[kGroup * kGroup];
  // Bands of 128 rows go out last-first, so the first rows' codes are the last written and the
  // likeliest to be cached when a weight gradient starts its reduction over the rows from the
  // first (interleaved A/B on dY of the gate+up layer step, 15 rounds: wgrad 1.4 us faster, in
  // 14 of them; the step 1.8 us).
  quant_dual_tile(x, ldx, qr, ldqr, sr, ld_sr, qc, ldqc, sc, ld_sc, blockIdx.x, gridDim.y - 1 - blockIdx.y, red, tile);
}

// ---------------------------------------------------------------------------------------------
// The forward pass's two quantisers in one launch: workgroups [0, nw) take the weight's 128x128
// tiles, the rest the activation's 128x128 tiles (both groupings). The two tensors are small next
// to a GEMM's operands (X [8192, 2048] is 32 MB): one launch fills the chip twice as long and
// pays the launch ramp once.
struct FwdQuantArgs {
  const uint16_t* x;
  int64_t ldx;
  uint8_t* qx;
  int64_t ldqx;
  float* sx;
  int64_t ld_sx;
  uint8_t* qxt;
  int64_t ldqxt;
  float* sxt;
  int64_t ld_sxt;
  int64_t x_col_groups;
  const uint16_t* w;
  int64_t ldw;
  uint8_t* qw;
  int64_t ldqw;
  uint8_t* qwt;
  int64_t ldqwt;
  float* sw;
  int64_t ld_sw;
  int64_t w_col_tiles, w_tiles;
};

__global__ __launch_bounds__(256) void quant_fwd_kernel(FwdQuantArgs a) {
  __shared__ __align__(16) uint32_t red[4][16][4];
  __shared__ __align__(16) uint8_t tile[kGroup * kGroup];
  const int64_t b = blockIdx.x;  // uniform branch per workgroup
  if (b < a.w_tiles) {
    quant_w_tile(a.w, a.ldw, a.qw, a.ldqw, a.qwt, a.ldqwt, a.sw, a.ld_sw, b / a.w_col_tiles, b % a.w_col_tiles,
                 &red[0][0][0], tile);
  } else {
    const int64_t bx = b - a.w_tiles;
    quant_dual_tile(a.x, a.ldx, a.qx, a.ldqx, a.sx, a.ld_sx, a.qxt, a.ldqxt, a.sxt, a.ld_sxt, bx % a.x_col_groups,
                    bx / a.x_col_groups, red, tile);
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_quant_rows(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, int64_t ldq,
                             float* dscale, int64_t ld_s, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerWG - 1) / kRowsPerWG), static_cast<unsigned>(cols / kGroup));
  hipLaunchKernelGGL(quant_rows_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x), rows, ldx,
                     static_cast<uint8_t*>(q), ldq, dscale, ld_s);
  return hipGetLastError();
}

hipError_t launch_quant_cols(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, int64_t ldq,
                             float* dscale, int64_t ld_s, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((cols + kColTile - 1) / kColTile), static_cast<unsigned>(rows / kGroup));
  hipLaunchKernelGGL(quant_cols_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x), cols, ldx,
                     static_cast<uint8_t*>(q), ldq, dscale, ld_s);
  return hipGetLastError();
}

hipError_t launch_quant_w(const void* w, int64_t n, int64_t k, int64_t ldw, void* q, int64_t ldq, void* qt,
                          int64_t ldqt, float* dscale, int64_t ld_s, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(k / kGroup), static_cast<unsigned>(n / kGroup));
  hipLaunchKernelGGL(quant_w_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(w), ldw,
                     static_cast<uint8_t*>(q), ldq, static_cast<uint8_t*>(qt), ldqt, dscale, ld_s);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, int64_t ldq_row,
                             float* dscale_row, int64_t ld_sr, void* q_col, int64_t ldq_col, float* dscale_col,
                             int64_t ld_sc, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(cols / kGroup), static_cast<unsigned>(rows / kGroup));
  hipLaunchKernelGGL(quant_dual_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x), ldx,
                     static_cast<uint8_t*>(q_row), ldq_row, dscale_row, ld_sr, static_cast<uint8_t*>(q_col), ldq_col,
                     dscale_col, ld_sc);
  return hipGetLastError();
}

hipError_t launch_quant_fwd(const void* x, int64_t m, int64_t k, int64_t ldx, void* qx, int64_t ldqx, float* sx,
                            int64_t ld_sx, void* qxt, int64_t ldqxt, float* sxt, int64_t ld_sxt, const void* w,
                            int64_t n, int64_t ldw, void* qw, int64_t ldqw, void* qwt, int64_t ldqwt, float* sw,
                            int64_t ld_sw, hipStream_t stream) {
  FwdQuantArgs a{static_cast<const uint16_t*>(x), ldx, static_cast<uint8_t*>(qx), ldqx, sx, ld_sx,
                 static_cast<uint8_t*>(qxt), ldqxt, sxt, ld_sxt, k / kGroup,
                 static_cast<const uint16_t*>(w), ldw, static_cast<uint8_t*>(qw), ldqw, static_cast<uint8_t*>(qwt),
                 ldqwt, sw, ld_sw, k / kGroup, (n / kGroup) * (k / kGroup)};
  const int64_t blocks = a.w_tiles + (m / kGroup) * (k / kGroup);
  hipLaunchKernelGGL(quant_fwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pf8
