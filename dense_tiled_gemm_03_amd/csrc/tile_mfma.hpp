#pragma once
// The tuned fp16 / bf16 tile kernel shared by the two operand layouts it
// serves (A row-major M x K, sak = 1):
//   B stored N x K (sbk = 1): the layout of the 4096 x 7168 x 16384 BF16
//     GEMM reported for the Ascend release in "Getting to know TileLang"
//     (six-piece section);
//   B stored K x N (sbn = 1): the row-major B of the first-GEMM listing of
//     "Getting to know TileLang".
//
// The structure is the tile loop of "TileKernels deep dive" section 3.1 and
// the first-GEMM listing of "Getting to know TileLang" (one output tile per
// workgroup, operand tiles staged in on-chip memory per K slice with a
// multi-stage pipeline, an fp32 accumulator copied to C once with a cast),
// laid out for gfx950:
//  - workgroup tile BM x BN (256 x 224 or 256 x 256), 4 waves in a 2 x 2
//    grid, each wave owning a (BM/2) x (BN/2) block of fp32 accumulators in
//    registers: 128 x 112 with 16x16x32 MFMAs, 128 x 128 with 32x32x16;
//  - K slice of 64: one LDS row is 128 bytes (eight 16-byte chunks); tiles
//    go HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging);
//    a ring of LDS stages per operand (Tile's A_ST, B_ST), the loads of the
//    next slices in flight while the current one is multiplied: 256 x 224
//    keeps two stages of A and three of B (148 KiB; a B line that misses L2
//    has two slices to arrive), 128 x 128 three of each when one workgroup
//    runs per CU, the others two of each;
//  - LDS chunk swizzle: chunk c of row r sits at chunk position
//    c ^ ((r >> 1) & 7); with it the ds_read_b128 patterns of both MFMA
//    shapes (rows l % 16 or l % 32, chunks by lane group) are free of bank
//    conflicts (measured with the LDS bank-conflict counter on gfx950; the
//    plain c ^ (r & 7) conflicts for one shape, c ^ (r & 7) ^ ((r >> 3) & 1)
//    for the other);
//  - each MFMA sub-step's fragments are read from LDS while the previous
//    sub-step's MFMAs run, one read issued after each MFMA (a wave can have
//    at most 15 LDS reads outstanding, and LDS latency under load is a few
//    hundred cycles, so reads are spread over the MFMA stream);
//  - edges: the buffer descriptor of each operand tile ends at the last valid
//    element, so rows past M (or N) read as zero; chunks past K get an
//    out-of-range offset and read as zero; the epilogue masks the stores;
//  - tile order: workgroups the hardware places on one XCD (blockIdx % 8)
//    get consecutive tile ids, walked in groups of GM M-tiles so concurrent
//    tiles on one XCD share A rows and B columns in that XCD's L2.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "fp8_codec.hpp"

namespace tg {
namespace tile {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int V> using Int = std::integral_constant<int, V>;

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every descriptor's range
constexpr int kXcds = 8;
// Workgroups of the eight-wave kernels that run at once: one per CU (their
// LDS rings take most of a CU's 160 KiB), 256 CUs.
constexpr int kRoundWgs = 256;

// MFMA shapes.  A fragment is DIM rows x KSTEP k of one operand; lane l
// supplies row (l % DIM) and the 16-byte chunk (l / DIM) of the sub-step's
// KSTEP-wide k range.  Accumulator element v of lane l is output row
// out_row(l, v), column l % DIM of the DIM x DIM block.
struct Mfma32 {
  static constexpr int DIM = 32, KSTEP = 16, NACC = 16;
  typedef f32x16 Acc;
  __device__ static int out_row(int l, int v) { return 8 * (v >> 2) + 4 * (l >> 5) + (v & 3); }
  template <typename T8>
  __device__ static Acc mma(T8 a, T8 b, Acc c) { return mfma32x32x16(a, b, c); }
};
struct Mfma16 {
  static constexpr int DIM = 16, KSTEP = 32, NACC = 4;
  typedef f32x4 Acc;
  __device__ static int out_row(int l, int v) { return 4 * (l >> 4) + v; }
  template <typename T8>
  __device__ static Acc mma(T8 a, T8 b, Acc c) { return mfma16x16x32(a, b, c); }
};

// A_ST / B_ST: LDS stages of the A and B operand tiles (at least 2 each).
// With S stages an operand's loads have S - 1 slices to arrive.
template <int BM_, int BN_, typename MMA_, int A_ST_ = 2, int B_ST_ = 2>
struct Tile {
  typedef MMA_ MMA;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int A_ST = A_ST_, B_ST = B_ST_;
  static constexpr int BK = 64;                      // k per LDS stage
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile (2 x 2 waves)
  static constexpr int FM = WTM / MMA::DIM, FN = WTN / MMA::DIM;
  static constexpr int SUBS = BK / MMA::KSTEP;       // MFMA sub-steps per slice
  static constexpr int ROW_BYTES = BK * 2;           // 128
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int LDS_BYTES = A_ST * A_BYTES + B_ST * B_BYTES;  // A stages, then B stages
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;  // 1 KiB loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int GM = 4;                       // M-tiles per tile-order group
  static_assert(WTM % MMA::DIM == 0 && WTN % MMA::DIM == 0, "wave tile must fit the MFMA");
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole loads per wave");
  static_assert(FM + FN <= 15, "a sub-step's reads must fit the lgkmcnt counter");
  static_assert(SUBS % 2 == 0, "fragment buffers alternate per sub-step");
  static_assert(A_ST >= 2 && B_ST >= 2, "at least two stages of each operand");
  static_assert(LDS_BYTES <= 160 * 1024, "stages must fit the LDS");
};

// s_waitcnt immediate (gfx9 layout): wait until at most `vm` vector-memory
// and `lgkm` LDS operations of this wave are outstanding; no expcnt wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return ((vm >> 4) & 3) << 14 | (lgkm & 15) << 8 | 7 << 4 | (vm & 15);
}

// Raw buffer descriptor over [base, base + bytes), as four scalar
// registers (base, stride 0, byte range, raw-buffer flags).  Every field is
// wave-uniform; readfirstlane says so and keeps it in SGPRs.
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFF));
  d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  d[3] = 0x00020000;
  return d;
}

// 16-byte-per-lane global -> LDS load (buffer_load_dwordx4 ... lds): lane l
// writes LDS bytes [lds + 16 l, lds + 16 l + 16), zeros when voff is out of
// the descriptor's range.  Issued as inline assembly so the compiler does
// not track it: each wave waits for its own loads with s_waitcnt vmcnt
// before the barrier that publishes them (the compiler's tracking would add
// vmcnt(0) waits in front of LDS transpose reads of other stages).  It has
// no register results, so no value the compiler sees is ever pending.  M0
// holds the LDS base; the s_nop covers the M0 -> LDS DMA hazard.  Nothing
// else in these kernels uses M0 (gfx950 LDS reads and MFMAs do not).
// `lds` is the 32-bit LDS byte address (wave-uniform).
__device__ __forceinline__ void load_lds16(const i32x4& desc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(desc) : "memory");
}

// The same load with the non-temporal cache policy (nt): for an operand that
// is read exactly once, so that streaming it through the XCD's L2 does not
// push out lines that other workgroups read again (the skinny kernel's B
// against its shared A).
__device__ __forceinline__ void load_lds16_nt(const i32x4& desc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(lds), "v"(voff), "s"(desc) : "memory");
}

// This workgroup's id with the ids of each XCD (the hardware places
// workgroup b on XCD b % 8) made contiguous.
__device__ __forceinline__ int xcd_id() {
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcds, local = b / kXcds;
  const int per = G / kXcds, rem = G % kXcds;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Tile id -> (tile row, tile column): groups of GM tile rows walked
// row-fastest.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int gm_size, int& tm,
                                        int& tn) {
  const int span = gm_size * tiles_n;
  const int group = id / span, first_m = group * gm_size;
  const int gm = min(gm_size, tiles_m - first_m);
  const int in = id - group * span;
  tm = first_m + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int gm_size, int& tm,
                                            int& tn) {
  tile_of(xcd_id(), tiles_m, tiles_n, gm_size, tm, tn);
}

// Grids with a partial last wave: workgroups for `full` whole tiles, then
// split units (each one split of a tile past the whole ones).  Workgroup b
// of G runs on XCD b % 8 as the b / 8-th of that XCD; every XCD takes its
// share of the whole tiles first and its share of the split units after
// them, so the split units fill the last wave on every XCD.  Ids stay
// contiguous per XCD.  Returns true and the tile id for a whole tile, false
// and the unit's index for a split unit.  (Each XCD's workgroup count is at
// least its share of whole tiles: G >= full.)
__host__ __device__ inline bool tail_unit(int b, int G, int full, int& id) {
  const int x = b % kXcds, l = b / kXcds;
  const int per = G / kXcds, rem = G % kXcds;
  const int fper = full / kXcds, frem = full % kXcds;
  const int fx = fper + (x < frem ? 1 : 0);                // whole tiles on XCD x
  const int before_f = x * fper + (x < frem ? x : frem);   // ... on the XCDs before x
  if (l < fx) {
    id = before_f + l;
    return true;
  }
  const int before = x * per + (x < rem ? x : rem);        // workgroups on the XCDs before x
  id = (before - before_f) + (l - fx);
  return false;
}

// Split of K across the workgroups of one tile: this workgroup's split of
// `splits`, the tile's id, and the scratch that combines the partial tiles
// (per-tile counters, fp32 partial tiles).  splits == 1: no split.
struct SplitK {
  int splits, split, tile;
  float* part;
  int* counters;
};

// fp8 output in place of C: e4m3fn codes Q (M x N bytes, row stride sqm) and
// one fp32 scale per 1 x 128 row slice, S[m * ssm + j * ssj] for slice j.
struct QuantOut {
  uint8_t* Q;
  int64_t sqm;
  float* S;
  int64_t ssm, ssj;
};

// Codes and scales of one accumulator block row (DIM rows x the wave's 128
// columns) of the quantising epilogue below.
template <bool FAST, bool FULL, typename MMA, int FN, typename Acc>
__device__ __forceinline__ void quant_store(const Acc (&acc)[FN], const float* sc, const float* rc,
                                            const bool* zero, const QuantOut& qo, int64_t M,
                                            int64_t N, int64_t row0, int64_t c, int64_t slice,
                                            int lane) {
#pragma unroll
  for (int v = 0; v < MMA::NACC; ++v) {
    const int64_t r = row0 + MMA::out_row(lane, v);
    if (FULL || r < M) {
      uint8_t* q = qo.Q + r * qo.sqm + c;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (FULL || c + j * MMA::DIM < N)
          q[j * MMA::DIM] = (uint8_t)(FAST ? code_of_fast(acc[j][v], sc[v], rc[v], zero[v])
                                           : code_of(acc[j][v], sc[v], zero[v]));
      if ((lane % MMA::DIM) == 0) qo.S[r * qo.ssm + slice * qo.ssj] = sc[v];
    }
  }
}

// One accumulator block row of the quantising epilogue: the row maxima over
// the wave's columns inside N -- the lane's FN accumulator blocks, then the
// DIM lanes that hold the row's other columns -- the scales, then the
// codes.  FULL: the wave's whole tile lies inside M x N.
template <bool FULL, typename MMA, int FN, typename Acc>
__device__ __forceinline__ void quant_block_row(const Acc (&acc)[FN], const QuantOut& qo, int64_t M,
                                                int64_t N, int64_t row0, int64_t c, int64_t slice,
                                                int lane) {
  float sc[MMA::NACC], rc[MMA::NACC];
  bool zero[MMA::NACC];
  bool fast = true;
#pragma unroll
  for (int v = 0; v < MMA::NACC; ++v) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < FN; ++j)
      if (FULL || c + j * MMA::DIM < N) m = fmaxf(m, fabsf(acc[j][v]));
#pragma unroll
    for (int o = 1; o < MMA::DIM; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    sc[v] = block_scale(m, zero[v]);
    rc[v] = 1.0f / sc[v];
    fast = fast && scale_in_fast_range(sc[v]);
  }
  // codes from x * (1 / s) with one correction when every scale of the
  // wave's rows allows it (wave-uniform), else by division
  if (__all(fast))
    quant_store<true, FULL, MMA>(acc, sc, rc, zero, qo, M, N, row0, c, slice, lane);
  else
    quant_store<false, FULL, MMA>(acc, sc, rc, zero, qo, M, N, row0, c, slice, lane);
}

template <bool FULL, typename MMA, int FM, int FN, typename Acc, int... Is>
__device__ __forceinline__ void quant_block_rows(Acc (&acc)[FM][FN], const QuantOut& qo, int64_t M,
                                                 int64_t N, int64_t row0, int64_t c, int64_t slice,
                                                 int lane, std::integer_sequence<int, Is...>) {
  // one call per block row, expanded at compile time: the accumulators are
  // only ever indexed by constants, so they stay in registers
  (quant_block_row<FULL, MMA>(acc[Is], qo, M, N, row0 + Is * MMA::DIM, c, slice, lane), ...);
}

// Quantising epilogue, for a wave tile 128 columns wide starting at a
// multiple of 128 (col0), so that each of its rows is one 1 x 128 slice: the
// fp32 accumulators go straight to codes, with no rounding to 16 bits first
// ("TileKernels deep dive" section 7.2: the fused kernel's result is
// quantised without being written back in a wider type).  Columns past N are
// left out of the row maxima explicitly: with B stored K x N their
// accumulators hold products with the next K row's first elements, not
// zeros.
template <typename MMA, int FM, int FN, typename Acc>
__device__ __forceinline__ void quant_epilogue(Acc (&acc)[FM][FN], const QuantOut& qo, int64_t M,
                                               int64_t N, int64_t row0, int64_t col0, int lane) {
  static_assert(FN * MMA::DIM == 128, "a wave row is one 1 x 128 slice");
  if (col0 >= N) return;  // the wave's slice lies past N (wave-uniform)
  const int64_t c = col0 + (lane % MMA::DIM), slice = col0 / 128;
  if (row0 + FM * MMA::DIM <= M && col0 + 128 <= N)
    quant_block_rows<true, MMA>(acc, qo, M, N, row0, c, slice, lane,
                                std::make_integer_sequence<int, FM>());
  else
    quant_block_rows<false, MMA>(acc, qo, M, N, row0, c, slice, lane,
                                 std::make_integer_sequence<int, FM>());
}

// Grouped products: the group of this workgroup's (XCD-contiguous) tile id
// -- the last group whose first tile id is not above it; groups with no rows
// hold no tiles -- and the tile's row and column inside the group, in
// groups of gm_size tile rows walked row-fastest.
__device__ __forceinline__ void group_coords(const GroupTable& gt, int bm, int gm_size, int& g,
                                             int& tm, int& tn) {
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcds, local = b / kXcds;
  const int per = G / kXcds, rem = G % kXcds;
  const int id = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  g = 0;
  while (g + 1 < gt.G && gt.tile0[g + 1] <= id) ++g;
  const int t = id - gt.tile0[g];
  const int tiles_m = (int)cdiv(gt.row0[g + 1] - gt.row0[g], bm);
  const int span = gm_size * gt.tiles_n;
  const int first_m = (t / span) * gm_size;
  const int gm = min(gm_size, tiles_m - first_m);
  const int in = t - (t / span) * span;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Split K: at most this many workgroups share one output tile.
constexpr int kMaxSplits = 8;

// Time, in waves of whole tiles over `cus` CUs, of a grid of `tiles` tiles
// of nk K slices each whose tiles past the first wave are split s ways
// (s = 1: no split): one wave, then ceil(tail * s / cus) waves of 1/s of a
// tile, plus the combine, which costs about two K slices per split past
// the first (the last split of a tile reads the others' partials).
inline double tail_waves(int64_t tiles, int64_t nk, int64_t cus, int s) {
  const int64_t whole = tiles / cus, tail = tiles % cus;
  if (s == 1 || tail == 0) return double((tiles + cus - 1) / cus);
  return double(whole) + double((tail * s + cus - 1) / cus) / s + 2.0 * (s - 1) / double(nk);
}

// Split count for the tiles past the first wave of a grid of more than one
// and less than two waves: the cheapest by tail_waves (the smallest on
// ties, 1 when nothing beats the unsplit grid) among those that leave every
// split at least 8 K slices.  Larger grids run unsplit: the chip is
// power-limited, so a partial last wave runs at a higher clock than a full
// one and loses less than its idle CUs suggest, and measured splits of the
// last of two or three waves gained nothing (4096 x 7168 x 16384 in
// 256 x 256 tiles, 6144 x 6144 x 4096), while one wave and a tail gained
// about 10% (4352 x 4096 x 4096: 158 us unsplit, 142 us with the 67 tiles
// past the first wave split 2 ways).
inline int tail_splits(int64_t tiles, int64_t nk, int64_t cus, int max_splits = kMaxSplits) {
  if (tiles <= cus || tiles >= 2 * cus) return 1;
  int best = 1;
  double best_w = tail_waves(tiles, nk, cus, 1);
  for (int s = 2; s <= max_splits && nk / s >= 8; ++s) {
    const double w = tail_waves(tiles, nk, cus, s);
    if (w < best_w) {
      best = s;
      best_w = w;
    }
  }
  return best;
}

// Float4s of a split's partial that one part of the combine loads per other
// split: the largest divisor of nq with at most `budget` float4s in flight
// per part across the S - 1 other splits.
constexpr int split_part_q(int nq, int s, int budget) {
  int c = budget / (s - 1);
  if (c < 1) c = 1;
  while (nq % c != 0) --c;
  return c;
}

// The tile's sum over its S split partials, in split order 0 .. S-1,
// starting from zero, into acc, which holds split `me`'s own partial on
// entry (so only the other S - 1 partials are read).  Partial float4 q of
// thread t (of THREADS) of split sp sits at float4 (sp * NQ + q) * THREADS + t of rp, written
// with device-coherent stores by the other splits.  The thread's NQ float4s
// go in parts of QP; each part's loads of every other split are issued
// unconditionally one part ahead of the additions, so the wait before a
// part's additions counts exactly the next part's loads.
template <int S, int THREADS, int BUDGET, int FM, int FN, typename Acc>
__device__ __forceinline__ void sum_splits(Acc (&acc)[FM][FN], __amdgpu_buffer_rsrc_t rp, int me,
                                           int t) {
  constexpr int NV = sizeof(Acc) / 16, NQ = FM * FN * NV;
  // two parts in flight next to the accumulators, at most BUDGET float4s
  // each (the registers the accumulators leave)
  constexpr int QP = split_part_q(NQ, S, BUDGET), NP = NQ / QP;
  f32x4 x[2][S - 1][QP];
  auto load_part = [&](f32x4(&dst)[S - 1][QP], int p) {
#pragma unroll
    for (int o = 0; o < S - 1; ++o) {
      const int sp = o + (o >= me ? 1 : 0);  // the o-th split other than me
#pragma unroll
      for (int u = 0; u < QP; ++u)
        dst[o][u] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rp, ((sp * NQ + p * QP + u) * THREADS + t) * 16, 0, 0x10));
    }
  };
  load_part(x[0], 0);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p + 1 < NP) load_part(x[(p + 1) & 1], p + 1);
    f32x4 s[QP];
#pragma unroll
    for (int u = 0; u < QP; ++u) s[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // splits before me, then mine, then those after me
#pragma unroll
    for (int o = 0; o < S - 1; ++o)
      if (o < me)
#pragma unroll
        for (int u = 0; u < QP; ++u) s[u] += x[p & 1][o][u];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int q = p * QP + u, c = q % NV, j = (q / NV) % FN, i = q / (NV * FN);
      s[u] += f32x4{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2],
                    acc[i][j][4 * c + 3]};
    }
#pragma unroll
    for (int o = 0; o < S - 1; ++o)
      if (o >= me)
#pragma unroll
        for (int u = 0; u < QP; ++u) s[u] += x[p & 1][o][u];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int q = p * QP + u, c = q % NV, j = (q / NV) % FN, i = q / (NV * FN);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][4 * c + e] = s[u][e];
    }
    // keep each part's loads in their part: the scheduler would otherwise
    // hoist later parts' loads and spill the registers they take
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The split-K combine at the end of a tile's K range: publish this split's
// fp32 partial tile -- accumulator float4 q of thread t at float4 index
// (split * NQ + q) * THREADS + t of the tile's slots, 16-byte runs
// contiguous across threads -- with device-coherent (sc1) stores; every wave
// waits for its stores before the barrier that precedes the tile's counter
// increment, so the split that finishes last reads every slot whole.  It
// adds the partials in split order (the result does not depend on which
// split finishes last) into acc, clears the counter and returns true; the
// other splits return false.  Every thread of the workgroup calls it.
// BUDGET: float4s of one part of the combine's loads (sum_splits).  S > 0:
// the split count is S (sk.splits == S), one instance of the sum; S == 0:
// a switch over sk.splits.  (Two or more instances of the sum in one
// kernel beside 112 accumulator registers spill thousands of VGPRs, though
// each alone fits; the eight-wave kernels take S from the host.)
template <int THREADS, int BUDGET, int S = 0, int FM, int FN, typename Acc>
__device__ __forceinline__ bool combine_splits(Acc (&acc)[FM][FN], const SplitK& sk, int t) {
  constexpr int NV = sizeof(Acc) / 16, NQ = FM * FN * NV;
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      sk.part + (int64_t)sk.tile * sk.splits * NQ * THREADS * 4, (short)0,
      sk.splits * NQ * THREADS * 16, 0x00020000);
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const f32x4 x = {acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2],
                         acc[i][j][4 * c + 3]};
        const int q = (i * FN + j) * NV + c;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rp,
                                               ((sk.split * NQ + q) * THREADS + t) * 16, 0, 0x10);
      }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int last;
  if (t == 0) last = atomicAdd(sk.counters + sk.tile, 1) == sk.splits - 1;
  __syncthreads();
  if (!last) return false;
  if constexpr (S > 0) {
    sum_splits<S, THREADS, BUDGET>(acc, rp, sk.split, t);
  } else {
  switch (sk.splits) {
    case 2: sum_splits<2, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    case 3: sum_splits<3, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    case 4: sum_splits<4, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    case 5: sum_splits<5, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    case 6: sum_splits<6, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    case 7: sum_splits<7, THREADS, BUDGET>(acc, rp, sk.split, t); break;
    default: sum_splits<kMaxSplits, THREADS, BUDGET>(acc, rp, sk.split, t); break;
  }
  }
  if (t == 0) __hip_atomic_store(sk.counters + sk.tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The LDS array of the tile stages: one per size, so that the bodies of one
// tile shape inlined into one kernel (whole and split tiles) share it.
template <int BYTES>
__device__ __forceinline__ char* tile_lds() {
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  return lds;
}

// One output tile (tile row tm, tile column tn) of C = A * B: the K loop
// and the epilogue.  BKN = false: B stored N x K (sbk = 1); true: B stored
// K x N (sbn = 1).
template <typename T, typename Cfg, bool BKN, bool SPLIT = false, bool QUANT = false>
__device__ __forceinline__ void tile_body(const GemmArgs& a, int tm, int tn,
                                          const SplitK& sk = SplitK{1, 0, 0, nullptr, nullptr},
                                          const QuantOut& qo = QuantOut{}) {
  typedef typename Elem<T>::x8 T8;
  typedef typename Cfg::MMA MMA;
  typedef typename MMA::Acc Acc;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUBS = Cfg::SUBS, DIM = MMA::DIM;
  char* const lds = tile_lds<Cfg::LDS_BYTES>();
  constexpr int A_ST = Cfg::A_ST, B_ST = Cfg::B_ST;
  // each slice's batch of loads starts with the shallower ring's
  constexpr bool A_FIRST = A_ST <= B_ST;
  // byte offsets of A stage s and B stage s in the LDS array
  auto a_off = [](int s) { return s * Cfg::A_BYTES; };
  auto b_off = [](int s) { return A_ST * Cfg::A_BYTES + s * Cfg::B_BYTES; };
  // the array's 32-bit LDS address, for the M0 operand of the LDS-direct loads
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = w >> 1, wn = w & 1;
  const int K = (int)a.K;
  // This workgroup's slices [kb0, kb1) of the K loop (all of them without a
  // split); loads at or past k_lim read zeros.
  static_assert(!(BKN && SPLIT), "split K takes B stored N x K");
  const int nk = (K + BK - 1) / BK;
  const int kb0 = SPLIT ? (int)((int64_t)sk.split * nk / sk.splits) : 0;
  const int kb1 = SPLIT ? (int)((int64_t)(sk.split + 1) * nk / sk.splits) : nk;
  const int k_lim = SPLIT ? min(K, kb1 * BK) : K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)(BKN ? a.sbk : a.sbn);

  // Operand tiles as buffer descriptors that end at the last valid element:
  // A rows m0 .. of length K; B rows n0 .. of length K (N x K), or B rows
  // 0 .. K-1 from column n0 (K x N).
  const int rows_a = (int)min<int64_t>(BM, a.M - m0), rows_b = (int)min<int64_t>(BN, a.N - n0);
  const T* Ab = static_cast<const T*>(a.A) + m0 * a.sam;
  const T* Bb = static_cast<const T*>(a.B) + (BKN ? n0 : n0 * a.sbn);
  const i32x4 ra = make_desc(Ab, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const i32x4 rb =
      make_desc(Bb, (uint32_t)(BKN ? ((K - 1) * ldb + rows_b) * 2 : ((rows_b - 1) * ldb + K) * 2));

  // Loads: wave w's i-th load fills LDS rows 8*(4i + w) .. +7 of a tile; lane
  // l writes row 8*(4i + w) + (l >> 3), chunk position l & 7, so it fetches
  // logical chunk (l & 7) ^ swizzle(row) = (l & 7) ^ (4 * (w & 1) + (l >> 4)).
  const int lrow = 8 * w + (lane >> 3);
  const int lchunk = (lane & 7) ^ (4 * (w & 1) + (lane >> 4));
  const uint32_t a_lane = (uint32_t)lrow * lda * 2 + 16 * lchunk;
  const uint32_t b_lane = (uint32_t)lrow * ldb * 2 + 16 * lchunk;
  const uint32_t a_step = 32 * lda * 2, b_step = 32 * ldb * 2;  // 32 rows per load index

  // K x N B: the stage holds B as [k][n] rows of BN * 2 bytes (BN = 256:
  // 32 chunks); chunk c of row k sits at position c ^ ((4k) & 31), which
  // keeps the transpose reads below free of bank conflicts.  Wave w's i-th
  // load fills k-rows 2 * (4i + w) and +1; lane l writes row 2 * (4i + w) +
  // (l >> 5), position l & 31, i.e. logical chunk (l & 31) ^ ((8w + 4 *
  // (l >> 5)) & 31).  Rows past K are fetched out of range (zeros).
  static_assert(!BKN || BN == 256, "K x N tiles are 256 columns wide");
  const int nrow = lane >> 5;
  const uint32_t nchunk = (lane & 31) ^ ((8 * w + 4 * nrow) & 31);
  const uint32_t nb_lane = (uint32_t)(2 * w + nrow) * ldb * 2 + 16 * nchunk;
  auto load_b = [&](uint32_t b_base, int i, int k0, bool kin) {
    const uint32_t dst = b_base + (4 * i + w) * 1024;
    if constexpr (BKN) {
      const bool rin = k0 + 8 * i + 2 * w + nrow < K;
      load_lds16(rb, dst, rin ? nb_lane + (uint32_t)(8 * i + k0) * ldb * 2 : kOutOfRange);
    } else {
      load_lds16(rb, dst, kin ? b_lane + i * b_step + 2 * k0 : kOutOfRange);
    }
  };

  auto load_a_stage = [&](int sa, int k0) {
    const bool kin = k0 + 8 * lchunk < k_lim;
    const uint32_t base = lds32 + a_off(sa);
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      load_lds16(ra, base + (4 * i + w) * 1024, kin ? a_lane + i * a_step + 2 * k0 : kOutOfRange);
  };
  auto load_b_stage = [&](int sb, int k0) {
    const bool kin = k0 + 8 * lchunk < k_lim;
    const uint32_t base = lds32 + b_off(sb);
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) load_b(base, i, k0, kin);
  };

  // Reads: fragment row r = (DIM-aligned base) + (l % DIM), chunk
  // s * (KSTEP / 8) + l / DIM of the 64-wide slice for sub-step s, at chunk
  // position chunk ^ swizzle(r) = chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  const int rd_lane = (lane % DIM) * Cfg::ROW_BYTES;
  const int rd_chunk = lane / DIM;
  const int a_rd = wm * Cfg::WTM * Cfg::ROW_BYTES + rd_lane;
  const int b_rd = wn * Cfg::WTN * Cfg::ROW_BYTES + rd_lane;  // within a B stage

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < MMA::NACC; ++v) acc[i][j][v] = 0.0f;

  // K x N B fragments come from ds_read_b64_tr_b16 (transpose read, gfx950):
  // within each 16-lane group, lane 4r + q supplies the address of 4
  // consecutive columns n0 + 4q .. +3 of k-row k0 + r, and lane i receives
  // column n0 + i of those 4 rows.  So lane l of group u = l / 16 points at
  // row s * KSTEP + 8 * kg + 4h + r, column nbase + nsub + 4q, with kg and
  // nsub the MFMA's k-group and column half of that lane group (32x32x16:
  // kg = u >> 1, nsub = 16 (u & 1); 16x16x32: kg = u, nsub = 0); two reads
  // (h = 0, 1) give the lane's 8 k-values.  Per lane and fragment the offset
  // does not depend on the sub-step or slice: precomputed for both h.
  constexpr int BROW = BN * 2;
  int kn_off[FN][2];
  if constexpr (BKN) {
    const int u = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
    const int kg = DIM == 32 ? u >> 1 : u, nsub = DIM == 32 ? 16 * (u & 1) : 0;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = 8 * kg + 4 * h + r;          // row within the sub-step
        const int nbase = wn * Cfg::WTN + j * DIM;  // multiple of 16
        const int chunk = (((nbase + nsub) >> 3) ^ ((4 * kr) & 31)) + (q >> 1);
        kn_off[j][h] = kr * BROW + chunk * 16 + (q & 1) * 8;  // within a B stage
      }
  }
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  auto read_b_kn = [&](const char* stage_base, int sub, int j) {
    const char* p = stage_base + sub * MMA::KSTEP * BROW;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + kn_off[j][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + kn_off[j][1]));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(T8, v);
  };

  // Fragments of one sub-step, double-buffered.
  T8 fa[2][FM], fb[2][FN];
  constexpr int BR = BKN ? 2 : 1;                    // LDS reads per B fragment
  constexpr int NRD = FM + BR * FN;                  // LDS reads per sub-step
  constexpr int NLD = Cfg::A_LOADS + Cfg::B_LOADS;   // LDS-direct loads per slice
  static_assert(NRD <= FM * FN && NLD <= FM * FN, "one read and one load per MFMA");
  auto chunk_off = [&](int sub) { return ((sub * (MMA::KSTEP / 8) + rd_chunk) ^ sw) * 16; };
  // The r-th read of sub-step `sub` of stage st, in the order the MFMAs
  // consume fragments: a0, b0 .. b[FN-1], a1 .. a[FM-1] (a K x N B fragment
  // is a pair of reads, both issued at its first slot).
  auto read_one = [&](int buf, int sa, int sb, int sub, int r) {
    const char* abase = lds + a_off(sa) + chunk_off(sub);
    const char* bbase = lds + b_off(sb) + chunk_off(sub);
    if (r == 0) {
      fa[buf][0] = *reinterpret_cast<const T8*>(abase + a_rd);
    } else if (r <= BR * FN) {
      if constexpr (BKN) {
        if ((r - 1) % 2 == 0) fb[buf][(r - 1) / 2] = read_b_kn(lds + b_off(sb), sub, (r - 1) / 2);
      } else {
        fb[buf][r - 1] = *reinterpret_cast<const T8*>(bbase + b_rd + (r - 1) * DIM * Cfg::ROW_BYTES);
      }
    } else {
      fa[buf][r - BR * FN] =
          *reinterpret_cast<const T8*>(abase + a_rd + (r - BR * FN) * DIM * Cfg::ROW_BYTES);
    }
  };
  // keeps the scheduler from moving work across it (one wave per SIMD issues
  // everything in order, so the source order below is the issue order)
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // One sub-step: the MFMAs on fragment buffer `cur`; after the n-th MFMA,
  // the n-th read of the next sub-step (into buffer cur ^ 1, from A stage
  // nsa and B stage nsb) and, when LOADS, the LDS-direct loads of A at
  // k = ld_ka into A stage ld_sa and of B at k = ld_kb into B stage ld_sb
  // (the shallower ring's first; A's when both are as deep), spread over
  // the sub-step.  Spreading reads and loads over the MFMA stream hides their
  // issue cycles under MFMA execution and keeps at most one sub-step of
  // reads (<= 15, the lgkmcnt limit) in flight.
  auto substep = [&](auto loads_c, int cur, int nsa, int nsb, int nsub, int ld_sa, int ld_sb,
                     int ld_ka, int ld_kb) {
    constexpr bool LOADS = decltype(loads_c)::value;
    const bool kin_a = ld_ka + 8 * lchunk < k_lim, kin_b = ld_kb + 8 * lchunk < k_lim;
    const uint32_t ld_abase = lds32 + a_off(ld_sa), ld_bbase = lds32 + b_off(ld_sb);
#pragma unroll
    for (int n = 0; n < FM * FN; ++n) {
      const int i = n / FN, j = n % FN;
      acc[i][j] = MMA::mma(fa[cur][i], fb[cur][j], acc[i][j]);
      if (n < NRD) read_one(cur ^ 1, nsa, nsb, nsub, n);
      if constexpr (LOADS) {
        // load q goes after MFMA q * FM * FN / NLD: spread evenly, since a CU
        // moves 64 B per clock from L2 and a burst of loads would stall the
        // wave's issue (and with it the MFMAs) behind a full memory queue
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
          if (q * FM * FN / NLD != n) continue;
          constexpr int FIRST = A_FIRST ? Cfg::A_LOADS : Cfg::B_LOADS;
          const bool is_a = A_FIRST ? q < FIRST : q >= FIRST;
          const int qa = A_FIRST ? q : q - FIRST, qb = A_FIRST ? q - FIRST : q;
          if (is_a)
            load_lds16(ra, ld_abase + (4 * qa + w) * 1024,
                       kin_a ? a_lane + qa * a_step + 2 * ld_ka : kOutOfRange);
          else
            load_b(ld_bbase, qb, ld_kb, kin_b);
        }
      }
      fence();
    }
  };

  // Pipeline, per slice kt in A stage sa = kt mod A_ST and B stage
  // sb = kt mod B_ST (sub-steps s = 0 .. SUBS-1):
  //   s < SUBS-1: MFMAs of sub-step s | reads of sub-step s+1;
  //   then: wait for this wave's loads of slice kt+1 and barrier (after it,
  //     slice kt+1 is in LDS for every wave, and every wave's reads of
  //     stages sa, sb have returned -- the last sub-step needs them now);
  //   s = SUBS-1: MFMAs | reads of sub-step 0 of kt+1 | loads of A for
  //     slice kt+A_ST -> A stage sa and of B for slice kt+B_ST -> B stage sb.
  // Slice j's batch is the loads of the shallower ring (A when both are as
  // deep), then of the deeper one: A(j+A_ST) and B(j+B_ST).  The prologue
  // issues the batches j = -max(A_ST, B_ST) .. -1 the same way (the parts
  // with a slice >= 0).  At the wait of slice kt, the shallower operand's
  // slice kt+1 is in batch kt+1-S (S = its stage count, first in that
  // batch) and the deeper one's in the same batch after it when the rings
  // are as deep, else in an older batch; what may stay in flight is
  // everything issued after: the deeper operand's part of batch kt+1-S
  // when it is deeper, and the batches kt+2-S .. kt-1.  Before slice 0
  // likewise, with one more batch.
  // Slices at or past K are fetched with out-of-range offsets: they move no
  // data, fill the idle stage with zeros and keep the loop free of branches.
  constexpr int DEEP = A_ST > B_ST ? A_ST : B_ST, SHALLOW = A_ST > B_ST ? B_ST : A_ST;
#pragma unroll
  for (int j = -DEEP; j < 0; ++j) {
    if (A_FIRST) {
      if (j + A_ST >= 0) load_a_stage(j + A_ST, (kb0 + j + A_ST) * BK);
      if (j + B_ST >= 0) load_b_stage(j + B_ST, (kb0 + j + B_ST) * BK);
    } else {
      if (j + B_ST >= 0) load_b_stage(j + B_ST, (kb0 + j + B_ST) * BK);
      if (j + A_ST >= 0) load_a_stage(j + A_ST, (kb0 + j + A_ST) * BK);
    }
  }
  constexpr int DEEP_TAIL = A_ST == B_ST ? 0 : (A_ST > B_ST ? Cfg::A_LOADS : Cfg::B_LOADS);
  constexpr int INIT_WAIT = DEEP_TAIL + (SHALLOW - 1) * NLD;
  constexpr int LOOP_WAIT = DEEP_TAIL + (SHALLOW - 2) * NLD;
  static_assert(INIT_WAIT <= 63, "loads in flight must fit the vmcnt counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INIT_WAIT) : "memory");
  __syncthreads();
  {
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(0, 0, 0, 0, r);
  }
  int sa = 0, sb = 0;
  for (int kt = kb0; kt < kb1; ++kt) {
    const int nsa = sa + 1 == A_ST ? 0 : sa + 1, nsb = sb + 1 == B_ST ? 0 : sb + 1;
#pragma unroll
    for (int sub = 0; sub < SUBS - 1; ++sub) {
      fence();
      substep(std::false_type(), sub & 1, sa, sb, sub + 1, 0, 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOOP_WAIT) : "memory");
    __syncthreads();
    fence();
    substep(std::true_type(), (SUBS - 1) & 1, nsa, nsb, 0, sa, sb, (kt + A_ST) * BK,
            (kt + B_ST) * BK);
    sa = nsa;
    sb = nsb;
  }

  if constexpr (SPLIT) {
    // 16 float4s per part with 224 accumulator registers, 8 with 256
    constexpr int budget = Cfg::FM * Cfg::FN * (MMA::NACC / 4) > 56 ? 8 : 16;
    if (!combine_splits<256, budget>(acc, sk, (int)threadIdx.x)) return;
  }

  static_assert(!(SPLIT && QUANT), "the quantising epilogue takes whole-K tiles");
  if constexpr (QUANT) {
    quant_epilogue<MMA>(acc, qo, a.M, a.N, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, lane);
    return;
  }

  // Epilogue: round each accumulator to the output type and store it inside
  // M x N.
  T* C = static_cast<T*>(a.C);
  const int64_t row0 = m0 + wm * Cfg::WTM, col0 = n0 + wn * Cfg::WTN + (lane % DIM);
  if (m0 + BM <= a.M && n0 + BN <= a.N) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < MMA::NACC; ++v)
          C[(row0 + i * DIM + MMA::out_row(lane, v)) * a.scm + col0 + j * DIM] =
              to_out<T>(acc[i][j][v]);
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < MMA::NACC; ++v) {
          const int64_t row = row0 + i * DIM + MMA::out_row(lane, v), col = col0 + j * DIM;
          if (row < a.M && col < a.N) C[row * a.scm + col] = to_out<T>(acc[i][j][v]);
        }
  }
}

template <typename T, typename Cfg, bool BKN>
__global__ __launch_bounds__(256) void gemm16_tile(GemmArgs a, int tiles_m, int tiles_n) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  tile_body<T, Cfg, BKN>(a, tm, tn);
}

// fp8 output: the product quantised per 1 x 128 row slice in the epilogue
// (a 256 x 256 tile: each wave's 128 columns are one slice).
template <typename T, typename Cfg, bool BKN>
__global__ __launch_bounds__(256) void gemm16_tile_q8(GemmArgs a, int tiles_m, int tiles_n,
                                                      QuantOut qo) {
  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  tile_body<T, Cfg, BKN, false, true>(a, tm, tn, SplitK{1, 0, 0, nullptr, nullptr}, qo);
}

// Split K: `splits` consecutive workgroups per tile, each over its share of
// the K slices, combined through scratch (see SplitK): for products with too
// few tiles to fill the CUs.
template <typename T, typename Cfg>
__global__ __launch_bounds__(256) void gemm16_tile_splitk(GemmArgs a, int tiles_m, int tiles_n,
                                                          int splits, float* part, int* counters) {
  const int id = xcd_id();
  const int tile = id / splits;
  int tm, tn;
  tile_of(tile, tiles_m, tiles_n, Cfg::GM, tm, tn);
  tile_body<T, Cfg, false, true>(a, tm, tn, SplitK{splits, id % splits, tile, part, counters});
}

// Grids of one whole wave and a partial one: `full` whole tiles, then the
// remaining tiles split `splits` ways over K (workgroup order as in
// tail_unit), combined through scratch as in gemm16_tile_splitk (the partials
// and counters are indexed by the tile's place among the split ones).
template <typename T, typename Cfg>
__global__ __launch_bounds__(256) void gemm16_tile_tail(GemmArgs a, int tiles_m, int tiles_n,
                                                        int full, int splits, float* part,
                                                        int* counters) {
  int id;
  const bool whole = tail_unit(blockIdx.x, gridDim.x, full, id);
  int tm, tn;
  tile_of(whole ? id : full + id / splits, tiles_m, tiles_n, Cfg::GM, tm, tn);
  if (whole)
    tile_body<T, Cfg, false>(a, tm, tn);
  else
    tile_body<T, Cfg, false, true>(a, tm, tn,
                                   SplitK{splits, id % splits, id / splits, part, counters});
}

}  // namespace tile
}  // namespace tg
