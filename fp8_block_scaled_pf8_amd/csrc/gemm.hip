// Block-scaled FP8 GEMM for gfx950: D[i,j] = sum_kb sa(kb,i) sb(kb,j) sum_{k in kb} A[i,k] B[j,k].
//
// Method [paperlayer.ai summary, appendix C "Production Training Details", bullet "FP8
// implementation pipeline"; paper.rainbus.top summary, 方法步骤详情 step (3)]: forward, data-gradient
// and weight-gradient GEMMs take blockwise E4M3 operands; the product of the two block scales is
// applied once per 128-wide K block and the result accumulates in FP32 and is written as BF16.
//
// Three kernels, one code path each (gfx950 only):
//  * gemm_mx_kernel (the default): 256 threads = 4 waves in a 2x2 grid own a BM x BN tile of D.
//    Operands stream into a ring of five LDS stage buffers by direct-to-LDS buffer loads, and
//    v_mfma_scale_f32_32x32x64_f8f6f4 applies the block scales while it accumulates in FP32: the
//    scales are powers of two, so their exponent bytes are exact E8M0 scale operands (the gfx950
//    counterpart of a block-scaled tensor-core path). The BF16 tile leaves through LDS as whole
//    rows; an FP32 form writes (or adds to) an FP32 result. Details above the kernel.
//  * gemm_mx_persistent_kernel: the same tiles and arithmetic, one workgroup per CU walking its
//    tiles with a ring of stage buffers that runs across tile boundaries (taken when every CU
//    gets two tiles or more, BF16 results, K a multiple of 256); with four tiles or more, half of
//    the workgroups start late so that the CUs' output bursts do not coincide.
//  * In both MX kernels the tiles of odd rounds walk K from its end (serpentine K), starting on
//    the K slices the previous round left in L2; a tile takes the same direction in either.
//  * gemm_promote_kernel: register-staged, double-buffered LDS; one v_mfma_f32_16x16x128_f8f6f4
//    covers a whole 128-wide scale block with a zero accumulator, and its FP32 partial is folded
//    into the running accumulator with one FMA by sa*sb per element.
//  * Both take B as the MFMA's first operand, so each lane owns consecutive output columns of
//    one row.
//  * Workgroup ids are remapped so each XCD (ids are dealt round-robin over 8) works on a
//    contiguous range of tiles, walked in groups of 8 tile-rows for L2 reuse of A and B panels.
#include "pf8_device.h"
#include "pf8_launch.h"

#include <atomic>
#include <type_traits>

namespace pf8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 for gfx9-family (dword data)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int e8m0_of(float s) { return static_cast<int>(__float_as_uint(s) >> 23) & 0xFF; }

__device__ __forceinline__ v8i lds_read32(const uint8_t* base, int off0, int off1) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + off0);
  const v4i hi = *reinterpret_cast<const v4i*>(base + off1);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// First (H = 0) or second (H = 1) 16 bytes of a 32-byte operand fragment, as 8 BF16 values.
template <int H>
__device__ __forceinline__ bf16x8 bf16_half(v8i v) {
  const v4i h = H == 0 ? v4i{v[0], v[1], v[2], v[3]} : v4i{v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(bf16x8, h);
}

// Store 4 consecutive BF16 outputs of row m starting at column n (masked at the ragged edges).
template <bool EDGE>
__device__ __forceinline__ void store4(uint16_t* __restrict__ d, int64_t ldd, int64_t m, int64_t n, int64_t M,
                                       int64_t N, float x0, float x1, float x2, float x3) {
  const uint32_t w0 = pack_bf16x2(x0, x1), w1 = pack_bf16x2(x2, x3);
  uint16_t* p = d + m * ldd + n;
  if (!EDGE) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
    return;
  }
  if (m >= M) return;
  if (n + 3 < N) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
  } else {
    if (n < N) p[0] = static_cast<uint16_t>(w0);
    if (n + 1 < N) p[1] = static_cast<uint16_t>(w0 >> 16);
    if (n + 2 < N) p[2] = static_cast<uint16_t>(w1);
  }
}

template <int BM, int BN, bool ROW_B, bool EDGE>
__global__ __launch_bounds__(256) void gemm_promote_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2;  // wave tile (2 x 2 waves)
  constexpr int A_BYTES = BM * kGroup, B_BYTES = BN * kGroup, STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM / 32, B_LOADS = BN / 32;  // 16-byte chunks per thread per K block
  __shared__ __align__(16) uint8_t smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile scheduling: XCD-contiguous ranges, then groups of 8 tile-rows ----
  int bid = blockIdx.x;
  {
    const int nb = gridDim.x, xcd = bid & 7, q = nb >> 3, rem = nb & 7;
    bid = xcd * q + min(xcd, rem) + (bid >> 3);
  }
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_grp = bid - grp * per_group;
  const int tm = first_m + in_grp % gsize;
  const int tn = in_grp / gsize;
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t M = p.m, N = p.n;
  const int nk = static_cast<int>(p.k / kGroup);

  // ---- global -> register loads ----
  // Full tiles put the per-chunk row offset in the scalar offset (one lane offset for all loads).
  // Edge tiles keep every row offset in the lane offset, so the buffer range check (sized to the
  // valid rows) turns rows past the edge into zeros.
  const int ld_row = t >> 3, ld_chunk = t & 7;
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int rows_a = EDGE ? static_cast<int>(min64(BM, M - m0)) : BM;
  const int rows_b = EDGE ? static_cast<int>(min64(BN, N - n0)) : BN;
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a + m0 * p.lda), 0, rows_a * lda, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b + n0 * p.ldb), 0, rows_b * ldb, kBufferFlags);
  const int voff_a = ld_row * lda + ld_chunk * 16;
  const int voff_b = ld_row * ldb + ld_chunk * 16;
  const int lds_w = ld_row * kGroup + ((ld_chunk ^ (ld_row & 7)) << 4);

  v4i ra[A_LOADS], rb[B_LOADS];
  auto gload = [&](int kb) {
    const int kofs = kb * kGroup;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const auto v = EDGE ? __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, voff_a + 32 * i * lda, kofs, 0)
                          : __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, voff_a, 32 * i * lda + kofs, 0);
      ra[i] = __builtin_bit_cast(v4i, v);
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const auto v = EDGE ? __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b + 32 * i * ldb, kofs, 0)
                          : __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b, 32 * i * ldb + kofs, 0);
      rb[i] = __builtin_bit_cast(v4i, v);
    }
  };
  auto lds_store = [&](int stage) {
    uint8_t* sa = smem + stage * STAGE;
    uint8_t* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<v4i*>(sa + lds_w + i * 32 * kGroup) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<v4i*>(sb + lds_w + i * 32 * kGroup) = rb[i];
  };
  // scale of B's row j in K block kb
  auto b_scale_idx = [&](int kb, int64_t j) -> int64_t {
    if (EDGE) j = min64(j, N - 1);
    return ROW_B ? static_cast<int64_t>(kb) * p.sb_k + j * p.sb_n : (j >> 7) * p.sb_n + static_cast<int64_t>(kb) * p.sb_k;
  };
  auto a_scale_idx = [&](int kb, int64_t i) -> int64_t {
    if (EDGE) i = min64(i, M - 1);
    return static_cast<int64_t>(kb) * p.ld_as + i;
  };

  {
    // 16x16x128 MFMA per scale block + FP32 FMA
    constexpr int TM = WM / 16, TN = WN / 16;
    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int l16 = lane & 15, quarter = lane >> 4;
    const int64_t a_row0 = m0 + wm * WM + l16;
    const int64_t b_col0 = n0 + wn * WN + 4 * quarter;  // this lane's first output column in tile j = 0
    const int ra_row0 = wm * WM + l16, rb_row0 = wn * WN + l16;
    const int sw = l16 & 7;
    const int c0 = ((2 * quarter) ^ sw) << 4, c1 = ((2 * quarter + 1) ^ sw) << 4;
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int NB = ROW_B ? 4 : 1;  // B scales per lane and 16-column tile
    auto load_scales = [&](int kb, float (&sa_v)[TM], float (&sb_v)[TN][NB]) {
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_v[i] = p.a_dscale[a_scale_idx(kb, a_row0 + 16 * i)];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < NB; ++r) sb_v[j][r] = p.b_dscale[b_scale_idx(kb, b_col0 + 16 * j + r)];
    };

    float sa_v[TM], sb_v[TN][NB], sa_n[TM], sb_n[TN][NB];
    gload(0);
    load_scales(0, sa_v, sb_v);
    lds_store(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
      const bool more = kb + 1 < nk;
      if (more) {
        gload(kb + 1);
        load_scales(kb + 1, sa_n, sb_n);
      }
      const uint8_t* sa = smem + (kb & 1) * STAGE;
      const uint8_t* sb = sa + A_BYTES;
      v8i fa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = ra_row0 + 16 * i;
        fa[i] = lds_read32(sa, row * kGroup + c0, row * kGroup + c1);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = rb_row0 + 16 * j;
        const v8i fb = lds_read32(sb, row * kGroup + c0, row * kGroup + c1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa[i], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = __builtin_fmaf(part[r], sa_v[i] * sb_v[j][ROW_B ? r : 0], acc[i][j][r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) lds_store((kb + 1) & 1);
      __syncthreads();
      if (more) {
#pragma unroll
        for (int i = 0; i < TM; ++i) sa_v[i] = sa_n[i];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < NB; ++r) sb_v[j][r] = sb_n[j][r];
      }
    }
    // epilogue: lane owns D[m][n .. n+3], m = lane%16 of the tile, n = 4*(lane/16)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t m = m0 + wm * WM + 16 * i + l16;
        const int64_t n = b_col0 + 16 * j;
        store4<EDGE>(p.d, p.ldd, m, n, M, N, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
  }
}

// Scheduling pattern for NM MFMAs: the ND LDS reads and the NV vector-memory reads go out spread
// evenly between them (sched_group_barrier masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read).
// Bunching the refill loads behind the last few MFMAs fills the texture unit's queues and stalls
// the wave's instruction stream, matrix instructions included.
// Vector-memory operations of `cnt` consecutive stages whose first is odd (`odd`) or even: D
// direct-to-LDS loads each, plus SS scale loads in each even stage.
constexpr int stage_ops(int cnt, bool odd, int d, int ss) {
  int n = 0;
  for (int i = 0; i < cnt; ++i) n += d + ((odd ? 1 : 0) ^ (i & 1) ? 0 : ss);
  return n;
}

template <int NM, int NV, int ND, int X = 0>
__device__ __forceinline__ void interleave_groups() {
  if constexpr (X < NM) {
    constexpr int d = (ND * (X + 1)) / NM - (ND * X) / NM;
    constexpr int v = (NV * (X + 1)) / NM - (NV * X) / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    interleave_groups<NM, NV, ND, X + 1>();
  }
}

// =============================================================================================
// MX kernel: direct-to-LDS pipeline.
//
//  * K advances in 64-byte stages (one 32x32x64 MFMA k-step; two stages per 128-wide scale block).
//  * NST stage buffers, each its own LDS object, filled by buffer_load ... lds (16 bytes per lane,
//    no staging registers) NST-1 stages ahead of use. Each wave issues D = (BM + BN) / 64 such
//    loads per stage; a wave's load covers 16 rows x 64 bytes. With NST = 5 a 256x256 tile uses
//    all 160 KB of LDS: four stages (128 KB) are in flight while one is consumed.
//  * 64-byte LDS rows hold 4 chunks of 16 bytes; chunk c of row r sits at c ^ ((r >> 2) & 3). A
//    b128 operand read serves 16 lanes (16 consecutive rows, one chunk each) per pass over the 64
//    banks; with this swizzle those 16 chunks land in 16 distinct 4-bank groups.
//  * Per stage and wave: TM*TN MFMAs split in two halves; between them the wave waits until its own
//    loads of the next stage have landed and its operand reads are done (explicit s_waitcnt), meets
//    the others at s_barrier, starts refilling the buffer all waves have just finished reading, and
//    reads the next stage's operands into the other fragment set while the second half of the
//    MFMAs runs. The refill's A-operand loads go out in that second half, its scales and B-operand
//    loads in the first half of the next stage, so the texture unit sees a steady stream.
//  * Stage s lives in buffer (s - h) mod NST. With five buffers the main loop runs ten stages
//    per trip and h = (stage count - 5) mod 10 (a short head, one code path per h), so the loop and
//    the final five stages always start in buffer 0 on an odd stage. Every buffer access thereby
//    names a fixed LDS object, and every stage's parity is known at compile time.
//  * The block scales travel with the operands, one set per 128-wide K block: the even stage of
//    the block loads them into its buffer's scale registers when it is issued, NST stages before
//    use, and the odd stage reads the previous buffer's registers.
// BF16IN: the operands are BF16 instead of E4M3 codes and carry no scales (the plain BF16 GEMM
// kept for comparison); K, the pitches and the stage size are then counted in bytes, a 64-byte
// stage is 32 values, and each fragment pair feeds two v_mfma_f32_32x32x16_bf16 (its first and
// second 16 bytes hold K values {0..7, 16..23} and {8..15, 24..31} of the stage in both
// operands, so every product of the stage is formed exactly once).
template <int BM, int BN, bool ROW_B, bool EDGE, int NST, bool F32 = false, bool BF16IN = false>
__global__ __launch_bounds__(256) void gemm_mx_kernel(GemmArgs p, int tiles_m, int tiles_n, int slots) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_ST = BM * BK, ST = (BM + BN) * BK;
  constexpr int A_DMA = BM / 64, B_DMA = BN / 64, D = A_DMA + B_DMA;  // loads per wave per stage
  static_assert(NST == 2 || NST == 5, "two or five stage buffers");
  // at least four buffers: the epilogue stages the BM x BN output tile through them
  constexpr int NBUF = NST < 4 ? 4 : NST;
  __shared__ __align__(16) uint8_t buf0[ST];
  __shared__ __align__(16) uint8_t buf1[ST];
  __shared__ __align__(16) uint8_t buf2[ST];
  __shared__ __align__(16) uint8_t buf3[ST];
  __shared__ __align__(16) uint8_t buf4[NBUF > 4 ? ST : 16];
  // the epilogue stages the output tile through the stage buffers, RPB rows per buffer
  constexpr int RPB = (ST / (BN * 2)) < 64 ? (ST / (BN * 2)) : 64;
  static_assert((BM + RPB - 1) / RPB <= NBUF, "the output tile fits the stage buffers");

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: keeps LDS and buffer offsets scalar
  const int wm = wave >> 1, wn = wave & 1;

  int bid = blockIdx.x;
  {
    const int nb = gridDim.x, xcd = bid & 7, q = nb >> 3, rem = nb & 7;
    bid = xcd * q + min(xcd, rem) + (bid >> 3);
  }
  // Serpentine K: a tile of an odd round (its position in its XCD's sequence / slots, slots = the
  // XCD's CUs) walks K from the end, starting on the K slices the previous round left in L2.
  // The persistent kernel takes the same direction for the same tile, so the two sum every
  // element in the same order. slots = 0: always forward.
  const int rev = (!BF16IN && slots > 0) ? __builtin_amdgcn_readfirstlane(((blockIdx.x >> 3) / slots) & 1) : 0;
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_grp = bid - grp * per_group;
  // the divisions above run on the vector ALU; pin the (uniform) tile coordinates to scalars
  const int tm = __builtin_amdgcn_readfirstlane(first_m + in_grp % gsize);
  const int tn = __builtin_amdgcn_readfirstlane(in_grp / gsize);
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t M = p.m, N = p.n;
  const int ns = static_cast<int>(p.k / BK);  // stages: even, and >= 6 with five buffers (the launcher checks)

  auto bufs = [&](int u) -> uint8_t* {
    return u == 0 ? buf0 : u == 1 ? buf1 : u == 2 ? buf2 : u == 3 ? buf3 : buf4;
  };

  // ---- direct-to-LDS loads ----
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int rows_a = EDGE ? static_cast<int>(min64(BM, M - m0)) : BM;
  const int rows_b = EDGE ? static_cast<int>(min64(BN, N - n0)) : BN;
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a + m0 * p.lda), 0, rows_a * lda, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b + n0 * p.ldb), 0, rows_b * ldb, kBufferFlags);
  // lane -> (row i>>2 of the 16-row slab, LDS chunk i&3); it fetches the chunk that belongs there
  const int dma_row = lane >> 2;
  const int dma_chunk = (lane & 3) ^ ((dma_row >> 2) & 3);
  const int voff_a = dma_row * lda + dma_chunk * 16;
  const int voff_b = dma_row * ldb + dma_chunk * 16;

  // ---- block scales (raw fp32 bits; the E8M0 byte is bits 23..30), one set per stage buffer ----
  const int l32 = lane & 31, half = lane >> 5;
  int64_t a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = EDGE ? min64(m0 + wm * WM + 32 * i + l32, M - 1) : m0 + wm * WM + 32 * i + l32;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row[j] = EDGE ? min64(n0 + wn * WN + 32 * j + l32, N - 1) : n0 + wn * WN + 32 * j + l32;
  // With tile scales and WN dividing 128, a wave's columns lie in one 128-column tile, and one B
  // scale serves all j. In an edge tile the columns clamp to N-1, which is in that tile whenever
  // any of them is stored.
  constexpr bool B_ONE = !ROW_B && (128 % WN == 0);
  constexpr int SB = B_ONE ? 1 : TN;
  // The two stages of a 128-wide K block share one set of scales: the even stage loads it into
  // its buffer's scale registers, the odd stage reads the previous buffer's. A stage's parity is
  // known at compile time wherever it is issued or consumed (see the stage layout below), and a
  // wave issues D direct-to-LDS loads per stage plus SS scale loads in an even stage.
  constexpr int SS = BF16IN ? 0 : TM + SB;
  uint32_t sc_a[NBUF][TM], sc_b[NBUF][SB];
  auto load_scales = [&](int s, uint32_t (&sa)[TM], uint32_t (&sb)[SB]) {
    // The explicit vmcnt counts assume that exactly TM + SB loads go out here, in program order
    // with the direct-to-LDS loads around them. Every index therefore passes through an opaque
    // asm statement: the compiler can neither merge two loads whose addresses it proves equal
    // (known bits of clamped columns let it do so) nor hoist one above earlier loads.
    const int64_t kb = (rev ? ns - 1 - s : s) >> 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int64_t idx = kb * p.ld_as + a_row[i];
      asm volatile("" : "+v"(idx));
      sa[i] = __float_as_uint(p.a_dscale[idx]);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      int64_t idx = ROW_B ? kb * p.sb_k + b_row[j] * p.sb_n : (b_row[j] >> 7) * p.sb_n + kb * p.sb_k;
      asm volatile("" : "+v"(idx));
      sb[j] = __float_as_uint(p.b_dscale[idx]);
    }
  };

  // Loads of stage s into buffer u: part 0 = the A operand's direct-to-LDS loads, part 1 = the
  // stage's scales (an even stage's) and the B operand's loads.
  auto issue_part = [&](auto u_c, int s, auto part_c, auto even_c) {
    constexpr int part = decltype(part_c)::value;
    constexpr int u = decltype(u_c)::value;
    uint8_t* buf = bufs(u);
    if constexpr (!BF16IN && part != 0 && decltype(even_c)::value) load_scales(s, sc_a[u], sc_b[u]);
    const int kofs = (rev ? ns - 1 - s : s) * BK;
#pragma unroll
    for (int j = 0; j < (part == 1 ? 0 : A_DMA); ++j) {
      const int slab = wave + 4 * j;  // rows 16*slab .. +15 of the A tile
      auto* dst = (__attribute__((address_space(3))) void*)(buf + slab * 16 * BK);
      if (EDGE) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, dst, 16, voff_a + slab * 16 * lda, kofs, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, dst, 16, voff_a, slab * 16 * lda + kofs, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < (part == 0 ? 0 : B_DMA); ++j) {
      const int slab = wave + 4 * j;
      auto* dst = (__attribute__((address_space(3))) void*)(buf + A_ST + slab * 16 * BK);
      if (EDGE) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, dst, 16, voff_b + slab * 16 * ldb, kofs, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, dst, 16, voff_b, slab * 16 * ldb + kofs, 0, 0);
    }
  };
  using PA = std::integral_constant<int, 0>;
  using PB = std::integral_constant<int, 1>;
  // a whole stage in the order a split refill uses (A operand, then scales and B operand), so that
  // the prologue leaves the loads in flight in the same order as every later stage
  auto issue_stage = [&](auto u_c, int s, auto even_c) {
    issue_part(u_c, s, PA{}, even_c);
    issue_part(u_c, s, PB{}, even_c);
  };
  constexpr int VA = A_DMA;  // vector-memory operations of a refill's first part

  // ---- operand fragments: set f = (buffer index) & 1 ----
  const int sw = (l32 >> 2) & 3;
  const int fo0 = l32 * BK + (((2 * half) ^ sw) << 4), fo1 = l32 * BK + (((2 * half + 1) ^ sw) << 4);
  v8i fa[2][TM], fb[2][TN];
  auto read_frags_a = [&](const uint8_t* buf, v8i (&a)[TM], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i < i0 || i >= i1) continue;
      const int base = (wm * WM + 32 * i) * BK;
      a[i] = lds_read32(buf, base + fo0, base + fo1);
    }
  };
  auto read_frags_b = [&](const uint8_t* buf, v8i (&b)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int base = A_ST + (wn * WN + 32 * j) * BK;
      b[j] = lds_read32(buf, base + fo0, base + fo1);
    }
  };
  auto read_frags = [&](const uint8_t* buf, v8i (&a)[TM], v8i (&b)[TN]) {
    read_frags_a(buf, a, 0, TM);
    read_frags_b(buf, b);
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // s_waitcnt vmcnt(n) lgkmcnt(0) (no expcnt wait). Vector memory operations complete in issue
  // order, so vmcnt(n) with n = the operations issued after a stage's last load guarantees that
  // stage. n is capped at the counter's 63, which only waits longer.
#define PF8_WAIT_VM_LGKM0(n0)                                                                  \
  do {                                                                                         \
    constexpr int n_ = (n0) < 63 ? (n0) : 63;                                                  \
    __builtin_amdgcn_s_waitcnt((n_ & 0xF) | ((n_ >> 4) << 14) | (0x7 << 4) | (0x0 << 8));      \
  } while (0)

  // One stage: s = stage index, u = its buffer (compile-time). A refill of buffer u with stage
  // s + NST is split in two to spread the loads over a whole stage of MFMAs: with `refill` the
  // A-operand loads go out in this stage's second half; with `prev` this stage's first half sends
  // the scales and B-operand loads of the previous stage's refill (stage s - 1 + NST).
  // Stage s is odd (`odd_c`) or even; a stage without `refill_c` has `after_c` stages issued
  // after stage s+1 (the final stages of K).
  auto stage = [&](int s, auto u_c, auto refill_c, auto last_c, auto prev_c, auto odd_c, auto after_c) {
    constexpr int u = decltype(u_c)::value;
    constexpr bool refill = decltype(refill_c)::value;
    constexpr bool prev = decltype(prev_c)::value;
    constexpr bool last = decltype(last_c)::value;
    constexpr bool odd = decltype(odd_c)::value;
    constexpr int after = decltype(after_c)::value;
    constexpr int f = u & 1, un = (u + 1) % NST, fn = un & 1;
    // an odd stage's scales sit in the previous buffer's registers (loaded with the even stage)
    constexpr int us = odd ? (u + NST - 1) % NST : u;
    // the previous stage's refill (stage s - 1 + NST) is even when this stage is (NST odd), or when
    // this stage is odd (NST even)
    constexpr bool prev_even = (NST % 2 == 1) ? !odd : odd;
    // decode this stage's scales; the empty asm hands each raw value over opaquely so the decode
    // (and the wait for its load, issued NST stages ago) cannot be hoisted next to the load
    int sae[TM], sbe[TN];
    if constexpr (!BF16IN) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint32_t v = sc_a[us][i];
        asm volatile("" : "+v"(v));
        sae[i] = static_cast<int>(v >> 23);
      }
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        uint32_t v = sc_b[us][j];
        asm volatile("" : "+v"(v));
        sbe[j] = static_cast<int>(v >> 23);
      }
#pragma unroll
      for (int j = SB; j < TN; ++j) sbe[j] = sbe[0];
    }
    auto mfma_rows = [&](int i0, int i1) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i < i0 || i >= i1) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (BF16IN) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16_half<0>(fb[f][j]), bf16_half<0>(fa[f][i]),
                                                                acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16_half<1>(fb[f][j]), bf16_half<1>(fa[f][i]),
                                                                acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0,
                                                                        sbe[j], 0, sae[i]);
          }
        }
      }
    };
    // second part of the previous stage's refill (its buffer is free since the last barrier)
    if constexpr (prev)
      issue_part(std::integral_constant<int, (u + NST - 1) % NST>{}, s - 1 + NST, PB{},
                 std::integral_constant<bool, prev_even>{});
    mfma_rows(0, TM / 2);
    if constexpr (prev)  // loads between the MFMAs
      interleave_groups<(TM / 2) * TN * (BF16IN ? 2 : 1), B_DMA + (prev_even ? SS : 0), 0>();
    // the first half of the MFMAs stays ahead of the wait and barrier: it keeps the matrix core
    // busy while the waves line up
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!last) {
      // stages s+2 .. s+NST-1 may still be in flight (fewer near the end of K); stage s+2 has
      // this stage's parity
      constexpr int inflight = refill ? NST - 2 : (after < NST - 2 ? after : NST - 2);
      PF8_WAIT_VM_LGKM0(stage_ops(inflight, odd, D, SS));
      __builtin_amdgcn_s_barrier();
      if constexpr (refill) issue_part(u_c, s + NST, PA{}, std::false_type{});
      if constexpr (fn != f) read_frags(bufs(un), fa[fn], fb[fn]);
      else read_frags_a(bufs(un), fa[fn], 0, TM / 2);  // only A rows the first half no longer needs
    }
    mfma_rows(TM / 2, TM);
    if constexpr (!last) {
      if constexpr (fn != f) {
        // next-stage operand reads and the refill's A-operand loads between the MFMAs
        interleave_groups<(TM - TM / 2) * TN * (BF16IN ? 2 : 1), VA, 2 * (TM + TN)>();
      } else {
        // with an odd number of buffers the last one hands over to the same fragment set: the
        // remaining operands are read once the MFMAs above have consumed the registers
        read_frags_a(bufs(un), fa[fn], TM / 2, TM);
        read_frags_b(bufs(un), fb[fn]);
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using F = std::false_type;
  using T = std::true_type;
  // Stage layout. K has ns stages, and ns is even: a multiple of 128 FP8 values, or of 128 BF16
  // values in the BF16 kernel. With five buffers the main loop runs ten stages per trip, so every
  // stage's buffer and parity are compile-time constants of its position in the loop body. The
  // first h = (ns - 5) mod 10 stages (h odd) form the head, one code path per h, and the last five
  // form the tail. Stage s lives in buffer (s - h) mod 5, so the loop and the tail always start in
  // buffer 0 on an odd stage. With two buffers there is no head: stage s lives in buffer s mod 2,
  // which is also its parity.
  const int h = NST == 5 ? static_cast<int>((ns - 5) % 10) : 0;
  auto prologue = [&](auto h_c) {
    constexpr int H = decltype(h_c)::value;
    auto ub = [](auto k_c) { return std::integral_constant<int, ((decltype(k_c)::value - H) % NST + NST) % NST>{}; };
    // stages 0 .. NST-1, issued in stage order (the explicit waits count loads in that order); of
    // stage NST-1 only the A-operand part, stage 0 sends the rest like any refill's second part.
    // A scheduling fence after each stage keeps the compiler from moving one stage's scale loads
    // among another stage's loads, which would break the counts.
    issue_stage(ub(I0{}), 0, T{});
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NST == 2) {
      issue_part(ub(I1{}), 1, PA{}, F{});
      __builtin_amdgcn_sched_barrier(0);
      PF8_WAIT_VM_LGKM0(VA);
    } else {
      issue_stage(ub(I1{}), 1, F{});
      __builtin_amdgcn_sched_barrier(0);
      issue_stage(ub(I2{}), 2, T{});
      __builtin_amdgcn_sched_barrier(0);
      issue_stage(ub(I3{}), 3, F{});
      __builtin_amdgcn_sched_barrier(0);
      issue_part(ub(std::integral_constant<int, 4>{}), 4, PA{}, T{});
      __builtin_amdgcn_sched_barrier(0);
      PF8_WAIT_VM_LGKM0(stage_ops(3, true, D, SS) + VA);  // after stage 0: stages 1..3 and stage 4's A part
    }
    __builtin_amdgcn_s_barrier();
    constexpr int u0 = decltype(ub(I0{}))::value;
    read_frags(bufs(u0), fa[u0 & 1], fb[u0 & 1]);
    // head stages 0 .. H-1 (all refill: ns >= H + 5)
    auto head = [&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      if constexpr (J < H) stage(J, ub(j_c), T{}, F{}, T{}, std::integral_constant<bool, (J & 1) != 0>{}, I0{});
    };
    head(I0{});
    head(I1{});
    head(I2{});
    head(I3{});
    head(std::integral_constant<int, 4>{});
    head(std::integral_constant<int, 5>{});
    head(std::integral_constant<int, 6>{});
    head(std::integral_constant<int, 7>{});
    head(std::integral_constant<int, 8>{});
  };
  if constexpr (NST == 5) {
    switch (h) {
      case 1: prologue(I1{}); break;
      case 3: prologue(I3{}); break;
      case 5: prologue(std::integral_constant<int, 5>{}); break;
      case 7: prologue(std::integral_constant<int, 7>{}); break;
      default: prologue(std::integral_constant<int, 9>{}); break;
    }
  } else {
    prologue(I0{});
  }

  // ---- main loop and tail ----
  using OD = std::true_type;   // odd stage
  using EV = std::false_type;  // even stage
  auto U = [](auto k_c) { return std::integral_constant<int, decltype(k_c)::value % NST>{}; };
  int s = h;
  if constexpr (NST == 5) {
    for (; s < ns - 5; s += 10) {
      stage(s, U(I0{}), T{}, F{}, T{}, OD{}, I0{});
      stage(s + 1, U(I1{}), T{}, F{}, T{}, EV{}, I0{});
      stage(s + 2, U(I2{}), T{}, F{}, T{}, OD{}, I0{});
      stage(s + 3, U(I3{}), T{}, F{}, T{}, EV{}, I0{});
      stage(s + 4, U(std::integral_constant<int, 4>{}), T{}, F{}, T{}, OD{}, I0{});
      stage(s + 5, U(std::integral_constant<int, 5>{}), T{}, F{}, T{}, EV{}, I0{});
      stage(s + 6, U(std::integral_constant<int, 6>{}), T{}, F{}, T{}, OD{}, I0{});
      stage(s + 7, U(std::integral_constant<int, 7>{}), T{}, F{}, T{}, EV{}, I0{});
      stage(s + 8, U(std::integral_constant<int, 8>{}), T{}, F{}, T{}, OD{}, I0{});
      stage(s + 9, U(std::integral_constant<int, 9>{}), T{}, F{}, T{}, EV{}, I0{});
    }
    // last five stages: nothing left to fetch
    stage(s, I0{}, F{}, F{}, T{}, OD{}, I3{});
    stage(s + 1, I1{}, F{}, F{}, F{}, EV{}, I2{});
    stage(s + 2, I2{}, F{}, F{}, F{}, OD{}, I1{});
    stage(s + 3, I3{}, F{}, F{}, F{}, EV{}, I0{});
    stage(s + 4, std::integral_constant<int, 4>{}, F{}, T{}, F{}, OD{}, I0{});
  } else {
    for (; s < ns - 2; s += 2) {
      stage(s, I0{}, T{}, F{}, T{}, EV{}, I0{});
      stage(s + 1, I1{}, T{}, F{}, T{}, OD{}, I0{});
    }
    stage(s, I0{}, F{}, F{}, T{}, EV{}, I0{});
    stage(s + 1, I1{}, F{}, T{}, F{}, OD{}, I0{});
  }
#undef PF8_WAIT_VM_LGKM0

  if constexpr (F32) {
    // ---- epilogue, FP32 result: one 64-row slab at a time through LDS ----
    // Slab i holds rows wm*WM + 32i + (lane % 32) of both wave rows, staged as row r = wm*32 + lane%32;
    // each lane writes its 4 consecutive columns per accumulator quarter, then every thread moves
    // whole 16-byte chunks of whole rows (64 lanes cover a 1 KB row), so the read-modify-write of
    // the result is coalesced. The old values of a slab are loaded first: their latency overlaps the
    // staging. Chunk c of staged row r sits at c ^ (r mod FCH): conflict-free writes and reads.
    constexpr int FCH = BN / 4;                      // 16-byte chunks per FP32 row
    constexpr int FRP = BN * 4;                      // staged row pitch (bytes)
    constexpr int FRPB = ST / FRP;                   // staged rows per stage buffer
    static_assert((FCH & (FCH - 1)) == 0, "FP32 rows are a power-of-two number of chunks");
    static_assert((64 + FRPB - 1) / FRPB <= NBUF, "a 64-row FP32 slab fits the stage buffers");
    constexpr int PER_S = 64 * FCH / 256;            // chunks per thread and slab
    auto fphys = [](int r, int c) -> int { return c ^ (r & (FCH - 1)); };
    auto srow = [&](int r) -> uint8_t* {
      return bufs(static_cast<unsigned>(r) / FRPB) + (static_cast<unsigned>(r) % FRPB) * FRP;
    };
    // s_waitcnt lgkmcnt(0) only: this wave's LDS accesses are done, stores may stay in flight
    constexpr int kWaitLgkm = 0xF | (0x7 << 4) | (0x3 << 14);
    __builtin_amdgcn_s_barrier();  // every wave is done with the operand buffers
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float4 old[PER_S];
      if (p.accumulate) {
#pragma unroll
        for (int it = 0; it < PER_S; ++it) {
          const int q = t + 256 * it, r = q / FCH, c = q % FCH;
          const int64_t gm = m0 + (r >> 5) * WM + 32 * i + (r & 31), gn = n0 + 4 * c;
          const float* src = p.d32 + gm * p.ldd + gn;
          if (!EDGE || (gm < M && gn + 3 < N)) {
            old[it] = *reinterpret_cast<const float4*>(src);
          } else {
            float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gm < M && gn + e < N) w[e] = src[e];
            old[it] = make_float4(w[0], w[1], w[2], w[3]);
          }
        }
      }
      {
        const int r = wm * 32 + l32;
        uint8_t* rb = srow(r);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = (wn * WN + 32 * j + 8 * q4 + 4 * half) >> 2;
            *reinterpret_cast<float4*>(rb + fphys(r, c) * 16) =
                make_float4(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
          }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int it = 0; it < PER_S; ++it) {
        const int q = t + 256 * it, r = q / FCH, c = q % FCH;
        const int64_t gm = m0 + (r >> 5) * WM + 32 * i + (r & 31), gn = n0 + 4 * c;
        float4 v = *reinterpret_cast<const float4*>(srow(r) + fphys(r, c) * 16);
        if (p.accumulate) v = make_float4(old[it].x + v.x, old[it].y + v.y, old[it].z + v.z, old[it].w + v.w);
        float* dst = p.d32 + gm * p.ldd + gn;
        if (!EDGE || (gm < M && gn + 3 < N)) {
          *reinterpret_cast<float4*>(dst) = v;
        } else if (gm < M) {
          const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < N) dst[e] = w[e];
        }
      }
      // every wave has read this slab back before the next one is staged
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  // ---- epilogue: BF16 tile staged through LDS, then written as whole rows ----
  // Lane owns D[m][n .. n+3], m = lane%32 of the MFMA tile, n = 8*(r/4) + 4*(lane/32). Row m of the
  // tile goes to buffer m/RPB; its 16-byte chunk c sits at chunk phys(m, c) so that the 32 rows a
  // wave writes at once spread over the banks, and a wave then reads 16-byte chunks of whole rows
  // back and stores them contiguously (a 512-byte row per 32 lanes for BN = 256).
  constexpr int CH = BN / 8;  // 16-byte chunks per output row
  constexpr int RP = BN * 2;  // output row pitch in LDS (bytes)
  auto phys = [](int row, int c) -> int {
    if constexpr ((CH & (CH - 1)) == 0) return c ^ (row & (CH - 1));
    else return (c + row) % CH;
  };
  __builtin_amdgcn_s_barrier();  // every wave is done with the operand buffers
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * WM + 32 * i + l32;
    uint8_t* rb = bufs(static_cast<unsigned>(row) / RPB) + (static_cast<unsigned>(row) % RPB) * RP;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = (wn * WN + 32 * j + 8 * q4) >> 3;
        const uint32_t w0 = pack_bf16x2(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1]);
        const uint32_t w1 = pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
        *reinterpret_cast<uint2*>(rb + phys(row, c) * 16 + 8 * half) = make_uint2(w0, w1);
      }
  }
  __syncthreads();
  constexpr int PER_T = BM * CH / 256;  // chunks per thread
  if constexpr (!EDGE && (CH & (CH - 1)) == 0) {
    // whole tiles with power-of-two rows: buffer stores over the tile's rows, the lane's offset
    // fixed and the chunk's row offset uniform (no 64-bit address arithmetic per store)
    if (static_cast<int64_t>(BM) * p.ldd * 2 <= 0x7FFFFFFF) {
      const __amdgpu_buffer_rsrc_t rsrc_d = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint8_t*>(p.d + m0 * p.ldd + n0), 0, static_cast<int>(BM * p.ldd * 2), kBufferFlags);
      const int ldd2 = static_cast<int>(p.ldd * 2);
      const int vo = (t / CH) * ldd2 + 16 * (t % CH);
#pragma unroll
      for (int it = 0; it < PER_T; ++it) {
        const int q = t + 256 * it;
        const int row = q / CH, c = q % CH;
        const uint4 v = *reinterpret_cast<const uint4*>(bufs(static_cast<unsigned>(row) / RPB) +
                                                        (static_cast<unsigned>(row) % RPB) * RP + phys(row, c) * 16);
        const v4u nv = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(nv, rsrc_d, vo, (256 / CH) * it * ldd2, 2);  // 2: non-temporal
      }
      return;
    }
  }
#pragma unroll
  for (int it = 0; it < PER_T; ++it) {
    const int q = t + 256 * it;
    const int row = q / CH, c = q % CH;
    const uint4 v = *reinterpret_cast<const uint4*>(bufs(static_cast<unsigned>(row) / RPB) +
                                                    (static_cast<unsigned>(row) % RPB) * RP + phys(row, c) * 16);
    const int64_t m = m0 + row, n = n0 + 8 * c;
    uint16_t* dst = p.d + m * p.ldd + n;
    // non-temporal: the result does not stay in the caches, where the next kernel would pay for its
    // write-back (in the gate+up layer step: 680.7 -> 656.5 us, the dY quantiser 83.6 -> 70.6 us)
    const v4i nv = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
    if (!EDGE) {
      __builtin_nontemporal_store(nv, reinterpret_cast<v4i*>(dst));
    } else if (m < M) {
      if (n + 7 < N) {
        __builtin_nontemporal_store(nv, reinterpret_cast<v4i*>(dst));
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// The persistent kernel's output staging buffer is written and read back through inline asm. The
// compiler's wait insertion makes an LDS access that aliases none of the direct-to-LDS loads it
// tracks wait for all of them, which here would be the next tile's first stages; the explicit
// lgkmcnt waits and barriers around these accesses order them instead. The read waits for its
// own results inside the asm statement before handing them over.
__device__ __forceinline__ void stg_write8(uint32_t addr, uint32_t w0, uint32_t w1) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(make_uint2(w0, w1)) : "memory");
}

__device__ __forceinline__ void stg_read8x16(const uint32_t (&addr)[8], v4i (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %9\n"
      "ds_read_b128 %2, %10\n"
      "ds_read_b128 %3, %11\n"
      "ds_read_b128 %4, %12\n"
      "ds_read_b128 %5, %13\n"
      "ds_read_b128 %6, %14\n"
      "ds_read_b128 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]), "v"(addr[7])
      : "memory");
}

// =============================================================================================
// Persistent MX kernel: one workgroup per CU walks a fixed list of BM x 256 output tiles
// (BM = 256 or 192), BF16 result, M and N multiples of the tile, K a multiple of 256 (>= 512).
//
//  * The workgroup with id w runs on XCD w mod 8 and takes every (grid/8)-th tile of that XCD's
//    contiguous tile range, i.e. the same tiles, in the same order, as the one-tile-per-workgroup
//    kernel's rounds; its workgroups never wait for one another.
//  * K streams in 64-byte stages through a ring of four LDS buffers that runs on across tile
//    boundaries: the refills of a tile's last four stages fetch the next tile's first four (all
//    of them issued before the tile's output stores), so the next tile's operands arrive while the
//    result leaves, and no workgroup start or prologue separates the tiles. The last tile fetches
//    its own first stages again, so that every tile runs the same code; the kernel drains them.
//  * Stage s of every tile sits in buffer s mod 4 (K is a multiple of 256): buffer indices and
//    stage parities are compile-time constants of the position in a four-stage loop body. The
//    two stages of a 128-wide K block share one set of scale registers, loaded with the even one.
//  * The result leaves through a fifth LDS buffer of its own, one 64-row slab at a time: each
//    wave writes 32 rows of its accumulators as BF16, then every thread moves whole 16-byte
//    chunks of whole rows with non-temporal stores.
//  * The waits count loads exactly as in gemm_mx_kernel. The first three waits of a tile also
//    count the previous tile's stores, which were issued after the stages they wait for: loads
//    and stores complete in issue order, so those waits do not wait for the stores.
//  * The tile loop is rotated (tile 0's first stages come before it, every trip ends with the next
//    tile's first stages), so each wait has one compile-time count. Lane-dependent offsets are
//    recomputed at the top of every tile from an opaque copy of the thread id: hoisted out of the
//    tile loop, their many derived addresses would stay live and spill.
// Results are bitwise those of gemm_mx_kernel with the same tile: every output element sums the
// same products in the same order.
template <int BM, bool ROW_B>
__global__ __launch_bounds__(256) void gemm_mx_persistent_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  constexpr int BN = 256, BK = 64, NST = 4;
  static_assert(BM == 256 || BM == 192, "256 or 192 output rows per tile");
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_ST = BM * BK, ST = (BM + BN) * BK;
  constexpr int A_DMA = BM / 64, B_DMA = BN / 64, D = A_DMA + B_DMA;
  constexpr int SB = ROW_B ? TN : 1;  // tile scales: a wave's 128 columns lie in one 128-column tile
  constexpr int SS = TM + SB;         // scale loads of an even stage
  constexpr int RP = BN * 2;          // staged output row pitch (bytes)
  constexpr int CH = BN / 8;          // 16-byte chunks per output row
  constexpr int ST_STORES = (64 * RP) / (256 * 16);  // 16-byte stores per thread and 64-row slab
  constexpr int N_STORES = TM * ST_STORES;           // per thread and tile
  static_assert(ST_STORES == 8, "eight 16-byte chunks per thread and slab");
  __shared__ __align__(16) uint8_t buf0[ST];
  __shared__ __align__(16) uint8_t buf1[ST];
  __shared__ __align__(16) uint8_t buf2[ST];
  __shared__ __align__(16) uint8_t buf3[ST];
  // 512-byte aligned: a staged row's chunk offsets (bits 4..8) can be XORed into its base address
  __shared__ __align__(512) uint8_t stg[64 * RP];

  const int t0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t0 >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ns = static_cast<int>(p.k / BK);  // a multiple of 4, >= 8 (the launcher checks)

  // ---- this workgroup's tiles ----
  const int nb = tiles_m * tiles_n;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, slots = gridDim.x >> 3;
  const int q = nb >> 3, rem = nb & 7;
  const int xcd_tiles = q + (xcd < rem ? 1 : 0), xcd_base = xcd * q + min(xcd, rem);
  const int ntiles = slot < xcd_tiles ? (xcd_tiles - slot + slots - 1) / slots : 0;
  if (ntiles == 0) return;
  auto tile_origin = [&](int r, int64_t& m0, int64_t& n0) {
    const int bid = xcd_base + slot + slots * r;
    constexpr int kGroupM = 8;
    const int per_group = kGroupM * tiles_n;
    const int grp = bid / per_group;
    const int first_m = grp * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in_grp = bid - grp * per_group;
    const int tm = __builtin_amdgcn_readfirstlane(first_m + in_grp % gsize);
    const int tn = __builtin_amdgcn_readfirstlane(in_grp / gsize);
    m0 = static_cast<int64_t>(tm) * BM;
    n0 = static_cast<int64_t>(tn) * BN;
  };
  auto bufs = [&](int u) -> uint8_t* { return u == 0 ? buf0 : u == 1 ? buf1 : u == 2 ? buf2 : buf3; };

  // ---- lane offsets (recomputed per tile) ----
  int t = t0, lane = t0 & 63;
  int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  int voff_a = 0, voff_b = 0, l32 = 0, half = 0, fo0 = 0, fo1 = 0;
  auto refresh = [&]() {
    asm volatile("" : "+v"(t));
    asm volatile("" : "+s"(lda), "+s"(ldb));
    lane = t & 63;
    const int dma_row = lane >> 2;
    const int dma_chunk = (lane & 3) ^ ((dma_row >> 2) & 3);
    voff_a = dma_row * lda + dma_chunk * 16;
    voff_b = dma_row * ldb + dma_chunk * 16;
    l32 = lane & 31;
    half = lane >> 5;
    const int sw = (l32 >> 2) & 3;
    fo0 = l32 * BK + (((2 * half) ^ sw) << 4);
    fo1 = l32 * BK + (((2 * half + 1) ^ sw) << 4);
  };
  refresh();

  // ---- load state: the tile whose stages the refills fetch ----
  __amdgpu_buffer_rsrc_t rsrc_a, rsrc_b;
  int64_t a_row[TM], b_row[SB];
  int load_rev = 0;  // odd tiles walk K from the end (serpentine, as gemm_mx_kernel's odd rounds)
  auto set_load_tile = [&](int r) {
    load_rev = r & 1;
    int64_t m0, n0;
    tile_origin(r, m0, n0);
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a + m0 * p.lda), 0, BM * lda, kBufferFlags);
    rsrc_b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b + n0 * p.ldb), 0, BN * ldb, kBufferFlags);
#pragma unroll
    for (int i = 0; i < TM; ++i) a_row[i] = m0 + wm * WM + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < SB; ++j) b_row[j] = n0 + wn * WN + 32 * j + l32;
  };
  // scale registers: one set per even buffer (0 and 2); an odd stage reads the previous buffer's
  uint32_t sc_a[2][TM], sc_b[2][SB];
  auto load_scales = [&](int s, uint32_t (&sa)[TM], uint32_t (&sb)[SB]) {
    // the waits count exactly TM + SB loads here: opaque indices keep the compiler from merging
    // two of them or hoisting one above earlier loads (as in gemm_mx_kernel)
    const int64_t kb = (load_rev ? ns - 1 - s : s) >> 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int64_t idx = kb * p.ld_as + a_row[i];
      asm volatile("" : "+v"(idx));
      sa[i] = __float_as_uint(p.a_dscale[idx]);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      int64_t idx = ROW_B ? kb * p.sb_k + b_row[j] * p.sb_n : (b_row[j] >> 7) * p.sb_n + kb * p.sb_k;
      asm volatile("" : "+v"(idx));
      sb[j] = __float_as_uint(p.b_dscale[idx]);
    }
  };
  // loads of the load tile's stage s into buffer u = s mod 4: part 0 = the A operand, part 1 = the
  // scales (even stages) and the B operand
  auto issue_part = [&](auto u_c, int s, auto part_c) {
    constexpr int u = decltype(u_c)::value;
    constexpr int part = decltype(part_c)::value;
    uint8_t* buf = bufs(u);
    if constexpr (part == 1 && (u % 2 == 0)) load_scales(s, sc_a[u / 2], sc_b[u / 2]);
    const int kofs = (load_rev ? ns - 1 - s : s) * BK;
#pragma unroll
    for (int j = 0; j < (part == 0 ? A_DMA : 0); ++j) {
      const int slab = wave + 4 * j;
      auto* dst = (__attribute__((address_space(3))) void*)(buf + slab * 16 * BK);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, dst, 16, voff_a, slab * 16 * lda + kofs, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < (part == 1 ? B_DMA : 0); ++j) {
      const int slab = wave + 4 * j;
      auto* dst = (__attribute__((address_space(3))) void*)(buf + A_ST + slab * 16 * BK);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, dst, 16, voff_b, slab * 16 * ldb + kofs, 0, 0);
    }
  };
  using PA = std::integral_constant<int, 0>;
  using PB = std::integral_constant<int, 1>;

  // ---- operand fragments: set f = stage parity ----
  v8i fa[2][TM], fb[2][TN];
  auto read_frags = [&](const uint8_t* buf, v8i (&a)[TM], v8i (&b)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = lds_read32(buf, (wm * WM + 32 * i) * BK + fo0, (wm * WM + 32 * i) * BK + fo1);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = lds_read32(buf, A_ST + (wn * WN + 32 * j) * BK + fo0, A_ST + (wn * WN + 32 * j) * BK + fo1);
  };

  v16f acc[TM][TN];

#define PF8_WAIT_VM_LGKM0(n0)                                                                  \
  do {                                                                                         \
    constexpr int n_ = (n0) < 63 ? (n0) : 63;                                                  \
    __builtin_amdgcn_s_waitcnt((n_ & 0xF) | ((n_ >> 4) << 14) | (0x7 << 4) | (0x0 << 8));      \
  } while (0)

  // One stage at body position u (tile stage s with s mod 4 = u):
  //  PREV: the first half sends the scales and B loads of load-tile stage ps (into buffer u - 1)
  //  REFILL: the second half sends the A loads of load-tile stage rs (into buffer u); EARLYB: and
  //          its B loads too (a tile's last stage: the next tile's stage 3 then leaves before the
  //          output stores)
  //  SWITCH: before the refill the load tile becomes tile `next`
  //  ZERO: the tile's first stage: the MFMAs start from zero
  //  INF: stages issued after stage s + 1 that may still be in flight at the wait
  //  XTRA: vector-memory operations issued after stage s + 1 besides those stages (the previous
  //        tile's output stores)
  auto stage = [&](auto u_c, auto prev_c, int ps, auto refill_c, int rs, auto earlyb_c, auto switch_c, int next,
                   auto zero_c, auto inf_c, auto xtra_c) {
    constexpr int u = decltype(u_c)::value;
    constexpr bool prev = decltype(prev_c)::value, refill = decltype(refill_c)::value;
    constexpr bool earlyb = decltype(earlyb_c)::value, sw_tile = decltype(switch_c)::value;
    constexpr bool zero = decltype(zero_c)::value;
    constexpr int inf = decltype(inf_c)::value, xtra = decltype(xtra_c)::value;
    constexpr int f = u & 1, un = (u + 1) & 3, fn = un & 1;
    constexpr bool odd = (u & 1) != 0;
    constexpr int us = u / 2;  // this K block's scale registers (loaded with its even stage)
    int sae[TM], sbe[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      uint32_t v = sc_a[us][i];
      asm volatile("" : "+v"(v));
      sae[i] = static_cast<int>(v >> 23);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      uint32_t v = sc_b[us][j];
      asm volatile("" : "+v"(v));
      sbe[j] = static_cast<int>(v >> 23);
    }
#pragma unroll
    for (int j = SB; j < TN; ++j) sbe[j] = sbe[0];
    auto mfma_rows = [&](int i0, int i1) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i < i0 || i >= i1) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v16f c = zero ? v16f{} : acc[i][j];
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[f][j], fa[f][i], c, 0, 0, 0, sbe[j], 0, sae[i]);
        }
      }
    };
    // the stage PREV sends lives in buffer u - 1 and has the other parity
    if constexpr (prev) issue_part(std::integral_constant<int, (u + 3) & 3>{}, ps, PB{});
    mfma_rows(0, TM / 2);
    if constexpr (prev) interleave_groups<(TM / 2) * TN, B_DMA + (odd ? SS : 0), 0>();
    __builtin_amdgcn_sched_barrier(0);
    // stage s + 2 has this stage's parity, stage s + 3 the other
    constexpr int after = (inf >= 1 ? D + (odd ? 0 : SS) : 0) + (inf >= 2 ? D + (odd ? SS : 0) : 0);
    PF8_WAIT_VM_LGKM0(after + xtra);
    __builtin_amdgcn_s_barrier();
    if constexpr (sw_tile) set_load_tile(next);
    if constexpr (refill) issue_part(u_c, rs, PA{});
    if constexpr (earlyb) issue_part(u_c, rs, PB{});
    read_frags(bufs(un), fa[fn], fb[fn]);
    mfma_rows(TM / 2, TM);
    interleave_groups<(TM - TM / 2) * TN, (refill ? A_DMA : 0) + (earlyb ? B_DMA : 0), 2 * (TM + TN)>();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using F = std::false_type;
  using T = std::true_type;
  using XS = std::integral_constant<int, N_STORES>;

  // ---- prologue: tile 0's stages 0..3 ----
  set_load_tile(0);
  issue_part(I0{}, 0, PA{});
  issue_part(I0{}, 0, PB{});
  __builtin_amdgcn_sched_barrier(0);
  issue_part(I1{}, 1, PA{});
  issue_part(I1{}, 1, PB{});
  __builtin_amdgcn_sched_barrier(0);
  issue_part(I2{}, 2, PA{});
  issue_part(I2{}, 2, PB{});
  __builtin_amdgcn_sched_barrier(0);
  issue_part(I3{}, 3, PA{});
  issue_part(I3{}, 3, PB{});
  __builtin_amdgcn_sched_barrier(0);
  // Staggered start: with four tiles or more per workgroup, the odd slots of every XCD begin their
  // first MFMAs about a third of a tile (half a tile's MFMA cycles) after the even ones, once
  // their first stages are on the way. Every tile ends with a 128 KB burst of stores per CU; with
  // all CUs in step those bursts coincide (32 MB per round) and slow the epilogues and the loads
  // of the next tiles' first stages. Offset, each half of the CUs stores while the other half
  // computes.
  if (ntiles >= 4 && (slot & 1)) {
    for (int z = 0; z < ns; ++z) __builtin_amdgcn_s_sleep(TM * TN / 2);  // 64 * TM * TN / 2 cycles per stage
  }
  PF8_WAIT_VM_LGKM0(D + (D + SS) + D);  // after stage 0: stages 1, 2 and 3
  __builtin_amdgcn_s_barrier();
  read_frags(buf0, fa[0], fb[0]);

  // tile 0's first body (no stores before it)
  stage(I0{}, F{}, 0, T{}, 4, F{}, F{}, 0, T{}, I2{}, I0{});
  stage(I1{}, T{}, 4, T{}, 5, F{}, F{}, 0, F{}, I2{}, I0{});
  stage(I2{}, T{}, 5, T{}, 6, F{}, F{}, 0, F{}, I2{}, I0{});
  stage(I3{}, T{}, 6, T{}, 7, F{}, F{}, 0, F{}, I2{}, I0{});
  for (int r = 0;; ++r) {
    refresh();
    int s = 4;
    for (; s < ns - 4; s += 4) {
      stage(I0{}, T{}, s + 3, T{}, s + 4, F{}, F{}, 0, F{}, I2{}, I0{});
      stage(I1{}, T{}, s + 4, T{}, s + 5, F{}, F{}, 0, F{}, I2{}, I0{});
      stage(I2{}, T{}, s + 5, T{}, s + 6, F{}, F{}, 0, F{}, I2{}, I0{});
      stage(I3{}, T{}, s + 6, T{}, s + 7, F{}, F{}, 0, F{}, I2{}, I0{});
    }
    // last body: its refills fetch the next tile's stages 0..3
    const int next = r + 1 < ntiles ? r + 1 : r;
    stage(I0{}, T{}, s + 3, T{}, 0, F{}, T{}, next, F{}, I2{}, I0{});
    stage(I1{}, T{}, 0, T{}, 1, F{}, F{}, 0, F{}, I2{}, I0{});
    stage(I2{}, T{}, 1, T{}, 2, F{}, F{}, 0, F{}, I2{}, I0{});
    stage(I3{}, T{}, 2, T{}, 3, T{}, F{}, 0, F{}, I2{}, I0{});

    // ---- epilogue: slab i holds rows wm*WM + 32i + (lane % 32) of both wave rows, staged as row
    // sr = wm*32 + lane%32; chunk c of staged row sr sits at chunk c ^ (sr mod 32) ----
    int64_t m0, n0;
    tile_origin(r, m0, n0);
    constexpr int kWaitLgkm = 0xF | (0x7 << 4) | (0x3 << 14);  // lgkmcnt(0) only
    // staging writes: this lane's row sr = wm*32 + l32 of the slab and its chunks c = wn*16 + k
    // (k = 4j + q4), chunk c at c ^ l32: with a 512-byte aligned row the address is one XOR of k
    const uint32_t wbase = (lds_addr(stg) + (wm * 32 + l32) * RP + 8 * half) | (((wn * 16) ^ l32) << 4);
    // staging reads: thread t takes chunk t % 32 of rows t / 32 + 8 it, which sits at chunk slot
    // (t % 32) ^ (t / 32) ^ 8 (it % 4)
    const uint32_t rbase = (lds_addr(stg) + (t >> 5) * RP) | (((t & 31) ^ (t >> 5)) << 4);
    // stores: a buffer resource over the tile's rows; the lane's offset is fixed per tile, the
    // slab's and the chunk's row offsets are uniform
    const __amdgpu_buffer_rsrc_t rsrc_d = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint8_t*>(p.d + m0 * p.ldd + n0), 0, static_cast<int>(BM * p.ldd * 2), kBufferFlags);
    const int ldd2 = static_cast<int>(p.ldd * 2);
    const int vo = (t >> 5) * ldd2 + 16 * (t & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t w0 = pack_bf16x2(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1]);
          const uint32_t w1 = pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
          stg_write8(wbase ^ ((4 * j + q4) << 4), w0, w1);
        }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
      uint32_t ra[ST_STORES];
      v4i rv[ST_STORES];
#pragma unroll
      for (int it = 0; it < ST_STORES; ++it) ra[it] = (rbase + 8 * it * RP) ^ ((it & 3) << 7);
      stg_read8x16(ra, rv);
#pragma unroll
      for (int it = 0; it < ST_STORES; ++it) {
        // row (it / 4) * WM + 32 i + 8 (it % 4) + t / 32 of the tile
        const int so = ((it >> 2) * WM + 32 * i + 8 * (it & 3)) * ldd2;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, rv[it]), rsrc_d, vo, so, 2);
      }
      if (i + 1 < TM) {
        // every wave has read this slab back before the next one is staged
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        __builtin_amdgcn_s_barrier();
      }
    }
    if (r + 1 == ntiles) break;
    // the next tile's first body: all of its stage 3 came with the last refills (no PREV in
    // stage 0), and this tile's stores follow stages 1..3
    stage(I0{}, F{}, 0, T{}, 4, F{}, F{}, 0, T{}, I2{}, XS{});
    stage(I1{}, T{}, 4, T{}, 5, F{}, F{}, 0, F{}, I2{}, XS{});
    stage(I2{}, T{}, 5, T{}, 6, F{}, F{}, 0, F{}, I2{}, XS{});
    stage(I3{}, T{}, 6, T{}, 7, F{}, F{}, 0, F{}, I2{}, I0{});
  }
  // the last tile's extra fetch writes LDS: it lands before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);
#undef PF8_WAIT_VM_LGKM0
}

// CUs of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Launches the persistent kernel for BM x 256 tiles when it applies: a BF16 result, tiles that
// divide M and N, K a multiple of 256 with at least 8 stages, and at least two tiles per CU.
// Returns hipErrorNotSupported (nothing launched) otherwise.
template <int BM>
static hipError_t launch_persistent(const GemmArgs& args, bool row_b, hipStream_t stream) {
  if (args.d32 != nullptr || args.m % BM != 0 || args.n % 256 != 0 || args.k % 256 != 0 || args.k < 512)
    return hipErrorNotSupported;
  const int64_t tiles_m = args.m / BM, tiles_n = args.n / 256;
  const int grid = device_cus() / 8 * 8;
  if (grid < 8 || tiles_m * tiles_n < 2 * static_cast<int64_t>(grid)) return hipErrorNotSupported;
  if (static_cast<int64_t>(BM) * args.ldd * 2 > 0x7FFFFFFF) return hipErrorNotSupported;  // a tile's rows in one buffer range
  const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
  if (row_b)
    hipLaunchKernelGGL((gemm_mx_persistent_kernel<BM, true>), dim3(grid), dim3(256), 0, stream, args, tm, tn);
  else
    hipLaunchKernelGGL((gemm_mx_persistent_kernel<BM, false>), dim3(grid), dim3(256), 0, stream, args, tm, tn);
  return hipGetLastError();
}

template <int BM, int BN, bool ROW_B, bool MX>
static hipError_t launch_tile(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = static_cast<int>((args.m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((args.n + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n)), block(256);
  const bool edge = args.m % BM != 0 || args.n % BN != 0;
  const int slots = device_cus() / 8;  // one tile per CU and round
  if constexpr (MX) {
    // five stage buffers fit the 160 KB LDS for every tile shape here; K extents under five
    // stages take the two-buffer pipeline
    static_assert(5 * (BM + BN) * 64 <= 160 * 1024, "five stage buffers fit the LDS");
    const int64_t ns = args.k / 64;
    if (ns < 2 || ns % 2 != 0) return hipErrorInvalidValue;  // the stage layout needs whole K blocks
    // FP32 results (three tile shapes only): one edge-checked kernel per pipeline depth
    constexpr bool kF32Tile = (BM == 256 && BN == 256) || (BM == 192 && BN == 256) || (BM == 128 && BN == 128);
    if (args.d32 != nullptr) {
      if constexpr (kF32Tile) {
        if (ns >= 5) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, true, 5, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
        else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, true, 2, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
      } else {
        return hipErrorInvalidValue;  // not reached: the FP32 tile choice offers only the shapes above
      }
    } else if (edge) {
      if (ns >= 5) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, true, 5>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
      else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, true, 2>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
    } else {
      if (ns >= 5) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, false, 5>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
      else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, ROW_B, false, 2>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
    }
  } else {
    if (edge)
      hipLaunchKernelGGL((gemm_promote_kernel<BM, BN, ROW_B, true>), grid, block, 0, stream, args, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_promote_kernel<BM, BN, ROW_B, false>), grid, block, 0, stream, args, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <int BM, int BN, bool MX>
static hipError_t launch_tile(const GemmArgs& args, bool row_b, hipStream_t stream) {
  return row_b ? launch_tile<BM, BN, true, MX>(args, stream) : launch_tile<BM, BN, false, MX>(args, stream);
}

// Plain BF16 GEMM (comparison kernel): the MX pipeline on BF16 operands, 256x256 or 128x128 tiles.
// args.k, args.lda and args.ldb are in bytes here.
template <int BM, int BN>
static hipError_t launch_bf16_tile(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = static_cast<int>((args.m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((args.n + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n)), block(256);
  const bool edge = args.m % BM != 0 || args.n % BN != 0;
  const int slots = 0;  // the BF16 comparison GEMM walks K forward
  const int64_t ns = args.k / 64;
  if (ns < 2 || ns % 2 != 0) return hipErrorInvalidValue;  // the stage layout needs an even stage count
  if (edge) {
    if (ns >= 5) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, false, true, 5, false, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
    else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, false, true, 2, false, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
  } else {
    if (ns >= 5) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, false, false, 5, false, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
    else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, false, false, 2, false, true>), grid, block, 0, stream, args, tiles_m, tiles_n, slots);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& args, hipStream_t stream) {
  const int64_t t256 = ((args.m + 255) / 256) * ((args.n + 255) / 256);
  const int64_t t128 = ((args.m + 127) / 128) * ((args.n + 127) / 128);
  // same model as the FP8 tile choice: rounds of one tile per CU x tile area / efficiency
  const double c256 = static_cast<double>((t256 + 255) / 256) * 65536.0;
  const double c128 = static_cast<double>((t128 + 255) / 256) * 16384.0 / 0.7;
  return c256 <= c128 ? launch_bf16_tile<256, 256>(args, stream) : launch_bf16_tile<128, 128>(args, stream);
}

// Macro-tile choice (MX variant). A launch takes ceil(tiles / 256) rounds of one tile per CU, so
// its time is modelled as rounds x (tile area / relative per-flop efficiency of the tile shape),
// and the cheapest shape wins. Smaller tiles re-read more operand bytes per flop (efficiency
// below 1) but can fill the 256 CUs evenly: the 12288x2048 weight gradient is 384 tiles of
// 256x256 (1.5 rounds) but exactly 512 of 192x256 (2 rounds of 3/4 the work), the 2048x6144 one
// 192 tiles of 256x256 but 256 of 256x192. The PROMOTE variant keeps an extra FP32 partial per
// MFMA in flight and uses 256x128 tiles to stay within registers; it has no FP32-output form.
hipError_t launch_gemm(const GemmArgs& args, bool row_b_scale, bool mx, hipStream_t stream) {
  if (!mx) {
    if (args.m >= 256) return launch_tile<256, 128, false>(args, row_b_scale, stream);
    return launch_tile<128, 128, false>(args, row_b_scale, stream);
  }
  struct Shape {
    int bm, bn;
    double eff;
  };
  constexpr Shape kShapes[] = {{256, 256, 1.0}, {256, 192, 0.95}, {192, 256, 0.95}, {256, 128, 0.85}, {128, 128, 0.7}};
  const bool f32 = args.d32 != nullptr;  // FP32 results are built for shapes 0, 2 and 4
  int best = 0;
  double best_cost = 0.0;
  for (int i = 0; i < static_cast<int>(sizeof(kShapes) / sizeof(kShapes[0])); ++i) {
    if (f32 && (i == 1 || i == 3)) continue;
    const Shape& sh = kShapes[i];
    const int64_t tiles = ((args.m + sh.bm - 1) / sh.bm) * ((args.n + sh.bn - 1) / sh.bn);
    const double cost = static_cast<double>((tiles + 255) / 256) * sh.bm * sh.bn / sh.eff;
    if (i == 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  // two tiles or more per CU: the persistent kernel overlaps each tile's output with the next
  // tile's first loads
  if (best == 0 || best == 2) {
    const hipError_t e = best == 0 ? launch_persistent<256>(args, row_b_scale, stream)
                                   : launch_persistent<192>(args, row_b_scale, stream);
    if (e != hipErrorNotSupported) return e;
  }
  switch (best) {
    case 0: return launch_tile<256, 256, true>(args, row_b_scale, stream);
    case 1: return launch_tile<256, 192, true>(args, row_b_scale, stream);
    case 2: return launch_tile<192, 256, true>(args, row_b_scale, stream);
    case 3: return launch_tile<256, 128, true>(args, row_b_scale, stream);
    default: return launch_tile<128, 128, true>(args, row_b_scale, stream);
  }
}

}  // namespace pf8
