#pragma once
// Eight-wave "ping-pong" form of the tile kernel (A row-major M x K; B
// stored N x K, or K x N with 256 x 256 tiles): the same tile loop as tile_body in
// tile_mfma.hpp ("TileKernels deep dive" section 3.1; the first-GEMM listing
// of "Getting to know TileLang": one output tile per workgroup, operand
// tiles staged per K slice in a multi-stage pipeline, an fp32 accumulator
// cast to C once), with the work of each SIMD split between two waves that
// take turns:
//  - workgroup tile 256 x BN (BN = 224), 512 threads: waves 0-3 (group 0,
//    one per SIMD) own columns 0 .. BN/2 - 1 of the tile, waves 4-7 (group
//    1) the other half; wave q of a group owns rows 64q .. 64q + 63, i.e. a
//    64 x BN/2 block of fp32 accumulators (4 x 7 blocks of 16x16x32 MFMAs);
//  - time runs in intervals separated by workgroup barriers.  In each
//    interval one group multiplies a whole 64-wide K slice from registers
//    (56 MFMAs per wave, nothing else) while the other group reads the next
//    slice's fragments from LDS (22 ds_read_b128) and issues its share of
//    the LDS-direct loads of a later slice; the groups swap every interval
//    (group 1 runs one interval behind group 0), so each SIMD's matrix core
//    always has one wave with MFMAs to issue while the other waits on LDS,
//    memory or the barrier;
//  - LDS: the rings of the one-group kernel -- two stages of A (the tile's
//    256 rows, 128 bytes of k per row) and three of B -- with the same chunk
//    swizzle c ^ ((r >> 1) & 7) (conflict-free 16x16x32 fragment reads);
//    group 0 loads every A stage, one slice ahead of its use, group 1 every
//    B stage, two slices ahead;
//  - edges, descriptors, tile order and the epilogues (the cast to C, or
//    with 256 x 256 tiles the fp8 quantisation per 1 x 128 row slice) as in
//    tile_body.
//
// Interval t follows barrier t.  Group 0 reads slice j in interval 2j and
// multiplies it in 2j + 1; group 1 reads it in 2j + 1 and multiplies it in
// 2j + 2.  Slice j's stages are therefore free after barrier 2j + 2, which
// is when group 0 (interval 2j + 2) refills A stage j with slice j + 2 and
// group 1 (interval 2j + 3) refills B stage j with slice j + 3.  Before the
// barrier that precedes group 0's reads of slice j + 1 (barrier 2j + 2),
// group 0 waits for all its loads (A of slice j + 1) and group 1 for all
// but the last slice's (B of slice j + 1 done, j + 2 in flight).  Each
// group passes 2 nk + 1 barriers.
#include "tile_mfma.hpp"

namespace tg {
namespace tile {

template <int BN_>
struct PPTile {
  static constexpr int BM = 256, BN = BN_, BK = 64;
  static constexpr int WTM = 64, WTN = BN / 2;         // wave tile
  static constexpr int FM = WTM / 16, FN = WTN / 16;   // 16x16 blocks per wave
  static constexpr int SUBS = 2;                       // k32 sub-steps per slice
  static constexpr int ROW_BYTES = 128;
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int A_ST = 2, B_ST = 3;
  static constexpr int LDS_BYTES = A_ST * A_BYTES + B_ST * B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;  // per wave of group 0
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;  // per wave of group 1
  static constexpr int GM = 4;
  static_assert(WTN % 16 == 0, "wave tile columns in whole 16x16 blocks");
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole loads per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "stages must fit the LDS");
};

// BKN = false: B stored N x K (sbk = 1); true: B stored K x N (sbn = 1),
// staged as [k][n] rows and read with the gfx950 transpose read, as in
// tile_body (256 x 256 tiles only).
// SPLITS > 1: this workgroup runs split sk.split of SPLITS (== sk.splits)
// equal ranges of the K slices and the tile's partials are combined as in
// the four-wave kernel (combine_splits); N x K tiles only.
// SWIGLU (with QUANT, N x K, 256 x 256 tiles): the tile covers 128 output
// columns; B stage rows 0 .. 127 are those columns' rows of the gate weights
// (a.B) and rows 128 .. 255 the same rows of the up weights (`up`, same
// strides), so group 0 accumulates the gate product g and group 1 the up
// product u of the same C block; the epilogue hands u to group 0 through
// LDS, which quantises h = silu(g) u.
template <typename T, typename Cfg, bool QUANT = false, bool BKN = false, int SPLITS = 1,
          bool SWIGLU = false>
__device__ __forceinline__ void pp_body(const GemmArgs& a, int tm, int tn,
                                        const QuantOut& qo = QuantOut{},
                                        const SplitK& sk = SplitK{1, 0, 0, nullptr, nullptr},
                                        const void* up = nullptr) {
  typedef typename Elem<T>::x8 T8;
  typedef f32x4 Acc;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUBS = Cfg::SUBS;
  constexpr int A_ST = Cfg::A_ST, B_ST = Cfg::B_ST;
  constexpr bool SPLIT = SPLITS > 1;
  static_assert(!(SPLIT && (QUANT || BKN)), "split K runs N x K tiles with the plain epilogue");
  static_assert(!SWIGLU || (QUANT && !BKN && !SPLIT && BN == 256),
                "SwiGLU: N x K weights, 256 x 256 tiles, quantised output");
  char* const lds = tile_lds<Cfg::LDS_BYTES>();
  auto a_off = [](int s) { return s * Cfg::A_BYTES; };
  auto b_off = [](int s) { return A_ST * Cfg::A_BYTES + s * Cfg::B_BYTES; };
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  // first row and first (output) column of the tile
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * (SWIGLU ? BN / 2 : BN);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = w >> 2, q = w & 3;  // group, wave within the group (its SIMD)
  const int K = (int)a.K;
  // this workgroup's K slices [s_begin, s_end) and the end of its K range
  const int nk_all = (K + BK - 1) / BK;
  const int s_begin = SPLIT ? (int)((int64_t)sk.split * nk_all / SPLITS) : 0;
  const int s_end = SPLIT ? (int)((int64_t)(sk.split + 1) * nk_all / SPLITS) : nk_all;
  const int nk = s_end - s_begin;
  const int k_lo = s_begin * BK, k_end = min(K, s_end * BK);
  // Slice order: workgroups of odd dispatch rounds (kRoundWgs run at once)
  // take their slices from the top of the range down.  A round re-reads the
  // operand rows the round before streamed, and so starts with the ones that
  // round read last, which are still in the last-level cache.  slice_k(j) is
  // the first k of the j-th slice taken; past the range it is negative (the
  // loads read zeros).
  const bool down = (blockIdx.x / kRoundWgs) & 1;
  auto slice_k = [&](int j) { return j >= nk ? -BK : k_lo + (down ? nk - 1 - j : j) * BK; };
  static_assert(!BKN || BN == 256, "K x N tiles are 256 columns wide");
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)(BKN ? a.sbk : a.sbn);

  // Operand tiles as buffer descriptors that end at the last valid element:
  // A rows m0 .. of length K; B rows n0 .. of length K (N x K), or B rows
  // 0 .. K-1 from column n0 (K x N).
  // (SwiGLU: rb the gate weights' rows n0 .., rbu the up weights' rows n0 ..)
  const int rows_a = (int)min<int64_t>(BM, a.M - m0);
  const int rows_b = (int)min<int64_t>(SWIGLU ? BN / 2 : BN, a.N - n0);
  const T* Ab = static_cast<const T*>(a.A) + m0 * a.sam;
  const T* Bb = static_cast<const T*>(a.B) + (BKN ? n0 : n0 * a.sbn);
  const i32x4 ra = make_desc(Ab, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const i32x4 rb =
      make_desc(Bb, (uint32_t)(BKN ? ((K - 1) * ldb + rows_b) * 2 : ((rows_b - 1) * ldb + K) * 2));
  i32x4 rbu = rb;
  if constexpr (SWIGLU)
    rbu = make_desc(static_cast<const T*>(up) + n0 * a.sbn, (uint32_t)(((rows_b - 1) * ldb + K) * 2));

  // Loads: wave q's i-th load of a stage fills its rows 8 (4i + q) .. + 7;
  // lane l writes row 8 (4i + q) + (l >> 3) at chunk position l & 7, i.e.
  // logical chunk (l & 7) ^ (4 (q & 1) + (l >> 4)).
  const int lrow = 8 * q + (lane >> 3);
  const int lchunk = (lane & 7) ^ (4 * (q & 1) + (lane >> 4));
  const uint32_t ld = g == 0 ? lda : ldb;
  const uint32_t l_lane = (uint32_t)lrow * ld * 2 + 16 * lchunk;
  const uint32_t l_step = 32 * ld * 2;
  auto load_a = [&](int slot, int k0) {
    const bool kin = k0 >= 0 && k0 + 8 * lchunk < k_end;
    const uint32_t base = lds32 + a_off(slot) + q * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      load_lds16(ra, base + i * 4096, kin ? l_lane + i * l_step + 2 * k0 : kOutOfRange);
  };
  // K x N B: the stage holds the tile's 256 columns as four quarters of 64
  // columns, quarter Q at Q * 8 KiB, each 64 k-rows of 128 bytes (8 chunks of
  // 16 bytes); chunk c of k-row k sits at position c ^ 2 t(k), t(k) =
  // ((k >> 1) & 1) | (((k >> 3) & 1) << 1).  Every load fills 1 KiB: 8
  // consecutive k-rows of one quarter, 8 rows of 128 bytes from B as in the
  // N x K layout (a load over 2 k-rows of 512 bytes measured 6 % slower).
  // Wave q's i-th load fills quarter i & 3, k-rows 8 G .. + 7 with G = 2q +
  // (i >> 2); lane l writes k-row 8 G + (l >> 3) at position l & 7, i.e.
  // logical chunk (l & 7) ^ 2 t = (l & 7) ^ (2 ((l >> 4) & 1) + 4 (G & 1)).
  // k-rows past K are fetched out of range (zeros).
  uint32_t nb_lane[2] = {0u, 0u};
  if constexpr (BKN) {
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const uint32_t kr = 16 * q + 8 * hi + (lane >> 3);
      const uint32_t c = (lane & 7) ^ (2 * ((lane >> 4) & 1) + 4 * hi);
      nb_lane[hi] = kr * ldb * 2 + 16 * c;
    }
  }
  auto load_b = [&](int slot, int k0) {
    const bool kin = k0 >= 0 && k0 + 8 * lchunk < k_end;
    const uint32_t base = lds32 + b_off(slot) + q * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) {
      if constexpr (BKN) {
        const int hi = i >> 2, quarter = i & 3;
        const bool rin = k0 >= 0 && k0 + 16 * q + 8 * hi + (lane >> 3) < k_end;
        load_lds16(rb, lds32 + b_off(slot) + quarter * 8192 + (2 * q + hi) * 1024,
                   rin ? nb_lane[hi] + (uint32_t)k0 * ldb * 2 + quarter * 128 : kOutOfRange);
      } else if constexpr (SWIGLU) {
        // loads 0 .. B_LOADS/2 - 1 fill the gate half, the others the up half
        constexpr int H = Cfg::B_LOADS / 2;
        load_lds16(i < H ? rb : rbu, base + i * 4096,
                   kin ? l_lane + (i % H) * l_step + 2 * k0 : kOutOfRange);
      } else {
        load_lds16(rb, base + i * 4096, kin ? l_lane + i * l_step + 2 * k0 : kOutOfRange);
      }
    }
  };

  // Fragment reads (16x16x32): row (16-aligned base) + (l % 16), chunk
  // 4 s + l / 16 of the slice for sub-step s, at position chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  const int a_rd = (q * Cfg::WTM + (lane & 15)) * Cfg::ROW_BYTES;
  const int b_rd = (g * Cfg::WTN + (lane & 15)) * Cfg::ROW_BYTES;
  int ch[SUBS];
#pragma unroll
  for (int s = 0; s < SUBS; ++s) ch[s] = ((4 * s + (lane >> 4)) ^ sw) * 16;

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0.0f, 0.0f, 0.0f, 0.0f};
  // K x N B fragments (ds_read_b64_tr_b16, as in tile_body): within each
  // 16-lane group, lane 4r + q' supplies the address of columns 4q' .. +3 of
  // k-row r of a 4-row group, and lane i receives column i of those rows;
  // lane l of group u = l / 16 points at k-row k = 32 s + 8u + 4h + r of the
  // slice, columns 128 g + 16 j + 4q', and the two reads (h = 0, 1) give its
  // 8 k-values.  In the layout above that is quarter 2g + (j >> 2), chunk
  // 2 (j & 3) + (q' >> 1) and t(k) = ((r >> 1) & 1) | ((u & 1) << 1), so the
  // address within a stage is
  //   8 KiB (2g + (j >> 2)) + 128 k + 32 ((j & 3) ^ t) + 16 (q' >> 1) + 8 (q' & 1)
  // and bits 5-6 hold (j & 3) ^ t alone: the lane keeps kn_d = the address for
  // s = h = j = 0 and XORs 32 (j & 3) into the address after adding the
  // stage base, the sub-step, h and the quarter (all multiples of 512 bytes;
  // the XOR after the loop-varying stage base also keeps the compiler from
  // hoisting 16 offsets per lane into registers for the whole loop).  Each
  // half-wave's 32 lanes then read 32 distinct 8-byte pairs of banks (eight
  // k-rows: r & 1 picks the 128-byte half of the 256-byte bank row, t the
  // 32-byte group within it).
  constexpr int BROW = 128;
  uint32_t kn_d = 0u;
  if constexpr (BKN) {
    static_assert(Cfg::WTN == 128, "K x N tiles are 256 columns wide");
    const int u = lane >> 4, r = (lane >> 2) & 3, qq = lane & 3;
    const int t = ((r >> 1) & 1) | ((u & 1) << 1);
    kn_d = 16384 * g + (8 * u + r) * BROW + 32 * t + 16 * (qq >> 1) + 8 * (qq & 1);
  }
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto read_b_kn = [&](int stage, int sub, int j) {
    // multiples of 512 bytes: the stage base, the sub-step's 32 k-rows, the quarter
    const uint32_t base = lds32 + b_off(stage) + sub * 32 * BROW + 8192 * (j >> 2) + kn_d;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(uintptr_t)(base ^ (32u * (j & 3))));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(uintptr_t)((base + 4 * BROW) ^ (32u * (j & 3))));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(T8, v);
  };

  T8 fa[SUBS][FM], fb[SUBS][FN];
  auto read_slice = [&](int sa, int sb) {
    const char* ab = lds + a_off(sa) + a_rd;
    const char* bb = lds + b_off(sb) + b_rd;
#pragma unroll
    for (int s = 0; s < SUBS; ++s) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[s][i] = *reinterpret_cast<const T8*>(ab + i * 16 * Cfg::ROW_BYTES + ch[s]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BKN)
          fb[s][j] = read_b_kn(sb, s, j);
        else
          fb[s][j] = *reinterpret_cast<const T8*>(bb + j * 16 * Cfg::ROW_BYTES + ch[s]);
      }
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < SUBS; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(fa[s][i], fb[s][j], acc[i][j]);
  };
  // Workgroup barrier; the scheduling fences keep the compiler from moving
  // MFMAs or reads across it (the phases must stay whole).
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_lds = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  if (g == 0) {
    load_a(0, slice_k(0));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();                                   // 0
    int sa = 0, sb = 0;
    for (int j = 0; j < nk; ++j) {
      const int na = sa + 1 == A_ST ? 0 : sa + 1;
      load_a(na, slice_k(j + 1));                // slice j + 1 into slice j - 1's stage
      read_slice(sa, sb);
      wait_lds();
      barrier();                                 // 2j + 1
      multiply();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      barrier();                                 // 2j + 2
      sa = na;
      sb = sb + 1 == B_ST ? 0 : sb + 1;
    }
  } else {
    load_b(0, slice_k(0));
    load_b(1, slice_k(1));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Cfg::B_LOADS) : "memory");
    barrier();                                   // 0
    barrier();                                   // 1
    int sa = 0, sb = 0;
    for (int j = 0; j < nk; ++j) {
      const int nb2 = sb == 0 ? 2 : sb - 1;      // (j + 2) mod 3: slice j - 1's stage
      load_b(nb2, slice_k(j + 2));
      read_slice(sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(Cfg::B_LOADS) : "memory");
      barrier();                                 // 2j + 2
      multiply();
      if (j + 1 < nk) barrier();                 // 2j + 3
      sa = sa + 1 == A_ST ? 0 : sa + 1;
      sb = sb + 1 == B_ST ? 0 : sb + 1;
    }
    // the last B loads (slices past the range, zeros) land before the LDS is released
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if constexpr (SPLIT) {
    // 12 float4s per part beside the 112 accumulator registers
    if (!combine_splits<512, 12, SPLITS>(acc, sk, (int)threadIdx.x)) return;
  }

  if constexpr (SWIGLU) {
    // Group 1's up accumulators go to the group 0 wave on the same SIMD
    // (same rows and columns) through the LDS, which both loops have left
    // idle: every load has landed and every fragment read is done.  Slot of
    // wave q's accumulator (i, j, v): ((q FM + i) FN + j) 4 + v, 64 lanes of
    // 4 bytes each (128 KiB in all).
    static_assert(4 * FM * FN * 4 * 64 * 4 <= Cfg::LDS_BYTES, "the up tile fits the LDS");
    float* xch = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (g == 1) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) xch[(((q * FM + i) * FN + j) * 4 + v) * 64 + lane] = acc[i][j][v];
    }
    __syncthreads();
    if (g == 1) return;
    // h = silu(g) u = g u / (1 + e^-g): e^-g overflows to inf for very
    // negative g, which gives h = 0 with the sign of g u
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc[i][j][v];
          const float uv = xch[(((q * FM + i) * FN + j) * 4 + v) * 64 + lane];
          acc[i][j][v] = gv * uv / (1.0f + expf(-gv));
        }
  }

  if constexpr (QUANT) {
    // fp8 output: with 256 x 256 tiles each wave's 128 columns are one
    // 1 x 128 slice of C, quantised straight from the accumulators
    static_assert(Cfg::WTN == 128, "a wave row is one 1 x 128 slice");
    quant_epilogue<Mfma16>(acc, qo, a.M, a.N, m0 + q * Cfg::WTM, n0 + g * Cfg::WTN, lane);
    return;
  }

  // Epilogue: round each accumulator to the output type and store it inside
  // M x N (lane l holds column l % 16, rows 4 (l / 16) + v of each block).
  T* C = static_cast<T*>(a.C);
  const int64_t row0 = m0 + q * Cfg::WTM + 4 * (lane >> 4);
  const int64_t col0 = n0 + g * Cfg::WTN + (lane & 15);
  if (m0 + BM <= a.M && n0 + BN <= a.N) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          C[(row0 + i * 16 + v) * a.scm + col0 + j * 16] = to_out<T>(acc[i][j][v]);
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = row0 + i * 16 + v, col = col0 + j * 16;
          if (row < a.M && col < a.N) C[row * a.scm + col] = to_out<T>(acc[i][j][v]);
        }
  }
}

template <typename T, typename Cfg, bool BKN = false>
__global__ __launch_bounds__(512) void gemm16_pp(GemmArgs a, int tiles_m, int tiles_n) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  pp_body<T, Cfg, false, BKN>(a, tm, tn);
}

// Split K: `splits` consecutive workgroups per tile, each over its share of
// the K slices, combined through scratch (SplitK): for products with too few
// tiles to fill the CUs.
template <typename T, typename Cfg, int S>
__global__ __launch_bounds__(512) void gemm16_pp_splitk(GemmArgs a, int tiles_m, int tiles_n,
                                                        float* part, int* counters) {
  const int id = xcd_id();
  const int tile = id / S;
  int tm, tn;
  tile_of(tile, tiles_m, tiles_n, Cfg::GM, tm, tn);
  pp_body<T, Cfg, false, false, S>(a, tm, tn, QuantOut{}, SplitK{S, id % S, tile, part, counters});
}

// Grids of one whole wave and a partial one: `full` whole tiles, then the
// remaining tiles split `splits` ways over K (workgroup order as in
// tail_unit); the partials and counters are indexed by the tile's place
// among the split ones.  Both bodies share one LDS array (tile_lds).
template <typename T, typename Cfg, int S>
__global__ __launch_bounds__(512) void gemm16_pp_tail(GemmArgs a, int tiles_m, int tiles_n,
                                                      int full, float* part, int* counters) {
  int id;
  const bool whole = tail_unit(blockIdx.x, gridDim.x, full, id);
  int tm, tn;
  tile_of(whole ? id : full + id / S, tiles_m, tiles_n, Cfg::GM, tm, tn);
  if (whole)
    pp_body<T, Cfg>(a, tm, tn);
  else
    pp_body<T, Cfg, false, false, S>(a, tm, tn, QuantOut{},
                                     SplitK{S, id % S, id / S, part, counters});
}

// fp8 output (256 x 256 tiles): the product quantised per 1 x 128 row slice
// in the epilogue.
template <typename T, typename Cfg, bool BKN = false>
__global__ __launch_bounds__(512) void gemm16_pp_q8(GemmArgs a, int tiles_m, int tiles_n,
                                                    QuantOut qo) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  pp_body<T, Cfg, true, BKN>(a, tm, tn, qo);
}

// Fused SwiGLU with an fp8 output (256 x 256 tiles, each over 128 output
// columns: tiles_n = ceil(N / 128)): gate weights a.B, up weights `up`, both
// stored N x K with the same strides.
template <typename T, typename Cfg>
__global__ __launch_bounds__(512) void gemm16_pp_swiglu(GemmArgs a, int tiles_m, int tiles_n,
                                                        QuantOut qo, const void* up) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  pp_body<T, Cfg, true, false, 1, true>(a, tm, tn, qo, SplitK{1, 0, 0, nullptr, nullptr}, up);
}

}  // namespace tile
}  // namespace tg
