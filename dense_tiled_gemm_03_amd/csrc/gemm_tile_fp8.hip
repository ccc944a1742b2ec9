// Tuned fp8 block-scaled kernel: C (bf16) = A * B with OCP E4M3FN codes and
// fp32 scales, one per 1 x 128 slice of each A row and one per 128 x 128
// block of B, A row-major (M x K, sak = 1) and B stored N x K (sbk = 1).
// FP8 and block-scaled GEMM are among the TileLang examples ("Getting to
// know TileLang", operator-coverage section); the E4M3 format with
// scale = amax / 448 is the one of "TileKernels deep dive" sections 4.3 and
// 7.2.  The 128-wide K slice of the tile loop ("TileKernels deep dive"
// section 3.1) is exactly one scale block:
//   P = sum over the slice of e4m3(a) * e4m3(b)      (fp8 MFMA, fp32, exact
//                                                      products)
//   acc += (SA[i, kb] * SB[j / 128, kb]) * P          (one VALU FMA)
// and C = round_bf16(acc) once at the end.
//
// Layout (gfx950):
//  - workgroup tile 256 (M) x 128 (N), 8 waves (4 along M x 2 along N, two
//    per SIMD, so one wave's VALU fold-in runs while the other's MFMAs do),
//    each owning 64 x 64 fp32 accumulators in VGPRs as 4 x 4 blocks of
//    16 x 16;
//  - one v_mfma_scale_f32_16x16x128_f8f6f4 (unit block exponents) per
//    block and slice, blocks taken column by column; the fold-in of a block
//    runs three MFMAs after it (measured: 532 us on 4096 x 7168 x 16384,
//    against 537 with two, 545 with one and 534 with four);
//  - registers: the A fragments of two slices alternate; each B fragment is
//    re-read for the next slice right after its last use in this one (so a
//    wave fits in 256 VGPRs with no accumulation registers);
//  - LDS: a ring of A stages (the A tile, 256 rows x 128 bytes, and the
//    slice's 256 A-row scales) and a ring of B stages (the B tile, 128 x 128
//    bytes, and the tile's B scale), three of each (156 KiB), all filled by
//    LDS-direct loads (full 128-byte lines for A and B), two slices ahead of
//    use; every wave issues the same eight loads per slice in the same
//    places, so one wait count serves all waves (measured with two A stages
//    and three to five B stages: slower, A needs its depth here);
//  - fragment reads: lane l of a 16x16x128 operand supplies row l % 16 and
//    32 k-bytes; lane group g = l / 16 takes 16-byte chunks g and g + 4 of
//    the 128-byte row (A and B use the same k assignment, so the sum is the
//    same), which with the chunk swizzle c ^ ((r >> 1) & 7) are
//    bank-conflict free (the bf16 kernel's 16x16x32 patterns);
//  - edges as in the bf16 kernels: descriptors end at the last valid row,
//    chunks past K read as zero, stores are masked; rows past M read zero
//    scales.
#include "../../include/tg_gemm.h"

#include <initializer_list>
#include <type_traits>
#include <utility>

#include "tile_mfma.hpp"

namespace tg {
namespace {

using tile::kOutOfRange;
using tile::make_desc;
using tile::load_lds16;
using tile::waitcnt_imm;

constexpr int F_BM = 256, F_BN = 128, F_BK = 128;    // tile, k per slice (bytes)
constexpr int F_WAVES = 8;                            // 4 along M x 2 along N
constexpr int F_FM = 4, F_FN = 4;                     // 16x16 blocks per wave
constexpr int F_A_BYTES = F_BM * F_BK;                // 32 KiB
constexpr int F_B_BYTES = F_BN * F_BK;                // 16 KiB
// An A stage holds the A codes, then a scale area of 8 waves x 256 bytes
// whose first 1 KiB are the tile's 256 fp32 A-row scales (waves 0-3); a B
// stage the B codes, then the same kind of area with the B scale at wave 4's
// slot.  Each wave issues one scale load into each ring per slice (out of
// range, i.e. zeros into its own unread slot, where it has nothing to load),
// so every wave's batch has the same loads in the same places.
constexpr int F_SCALES = F_WAVES * 256;               // scale area of a stage
constexpr int F_ASTAGE = F_A_BYTES + F_SCALES;        // 34 KiB
constexpr int F_BSTAGE = F_B_BYTES + F_SCALES;        // 18 KiB
constexpr int F_A_LD = F_A_BYTES / 1024 / F_WAVES;    // 4 loads per wave
constexpr int F_B_LD = F_B_BYTES / 1024 / F_WAVES;    // 2 loads per wave
constexpr int F_APART = 1 + F_A_LD;                   // A-ring loads per wave per slice
constexpr int F_BPART = F_B_LD + 1;                   // B-ring loads per wave per slice
constexpr int F_NLD = F_APART + F_BPART;
constexpr int F_LAG = 3;                              // MFMAs between a block and its fold-in
constexpr int F_NMMA = F_FM * F_FN;                   // MFMAs per wave per slice
constexpr int F_AS = 3, F_BS = 3;                     // stages of the A and B rings

// Global -> LDS loads with a wave-uniform scalar offset: lane l reads
// [voff + soff, + 16) (or + 4) of the buffer into LDS bytes [lds + 16 l, + 16)
// (or [lds + 4 l, + 4)).  The range check is left to voff alone (on this
// architecture the scalar offset may be outside it): every lane that must
// read zeros gets an out-of-range voff, and an in-range voff plus the
// scalar offset (the slice's k) stays inside the row and chunk it names.
// Inline assembly for the same reason as the loads of tile_mfma.hpp;
// keeping the per-lane part to one register per load keeps the kernel
// within 256 VGPRs.
__device__ __forceinline__ void load_lds16s(const i32x4& desc, uint32_t lds, uint32_t voff,
                                            uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(desc), "s"(soff) : "memory");
}
__device__ __forceinline__ void load_lds4s(const i32x4& desc, uint32_t lds, uint32_t voff,
                                           uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(desc), "s"(soff) : "memory");
}

// One 256 x 128 output tile (tile row tm, tile column tn): the K loop and the
// epilogue.  AS / BS: stages of the A ring (A codes + A scales) and of the B
// ring (B codes + B scale); with S stages an operand's loads have S - 1
// slices to arrive.
// Kinds of wave by the scale load each issues per slice: the A-row scales
// (waves 0-3), the tile's B scale (wave 4), none (waves 5-7).  Each kind
// runs its own copy of the K loop, so its loads and wait counts are fixed
// at compile time and no branch splits the MFMA stream.
enum { kScaleA = 0, kScaleB = 1, kScaleNone = 2 };

// The LDS array of the stage rings, one per size, shared by the copies of
// the K loop inlined into one kernel.
template <int BYTES>
__device__ __forceinline__ char* fp8_lds() {
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  return lds;
}

template <int AS, int BS, int KIND>
__device__ __forceinline__ void fp8_tile_body(const GemmArgs& a, int tm, int tn) {
  static_assert(AS >= 2 && BS >= AS, "at least two stages, B at least as deep as A");
  static_assert(AS * F_ASTAGE + BS * F_BSTAGE <= 160 * 1024, "LDS");
  char* const lds = fp8_lds<AS * F_ASTAGE + BS * F_BSTAGE>();
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
  // byte offsets of A stage s and B stage s
  auto a_off = [](int st) { return st * F_ASTAGE; };
  auto b_off = [](int st) { return AS * F_ASTAGE + st * F_BSTAGE; };

  const int64_t m0 = (int64_t)tm * F_BM, n0 = (int64_t)tn * F_BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w & 3, wn = w >> 2;
  const int K = (int)a.K;
  const int nkb = (K + F_BK - 1) / F_BK;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;

  const int rows_a = (int)min<int64_t>(F_BM, a.M - m0), rows_b = (int)min<int64_t>(F_BN, a.N - n0);
  const uint8_t* Ab = static_cast<const uint8_t*>(a.A) + m0 * a.sam;
  const uint8_t* Bb = static_cast<const uint8_t*>(a.B) + n0 * a.sbn;
  const i32x4 ra = make_desc(Ab, (uint32_t)((rows_a - 1) * lda + K));
  const i32x4 rb = make_desc(Bb, (uint32_t)((rows_b - 1) * ldb + K));
  // A scales of rows m0 ..: SA[i, kb] at (i * ssam + kb * ssak) floats; the
  // tile's B scale row SB[n0 / 128, kb] at kb * ssbk floats
  const float* SAb = a.SA + m0 * a.ssam;
  const float* SBb = a.SB + (n0 / 128) * a.ssbn;
  const i32x4 rsa = make_desc(SAb, (uint32_t)(((rows_a - 1) * a.ssam + (nkb - 1) * a.ssak + 1) * 4));
  const i32x4 rsb = make_desc(SBb, (uint32_t)(((nkb - 1) * a.ssbk + 1) * 4));

  // Loads of a slice (k0 bytes in): the tile's 8-row groups g = w + 8 q of A
  // (q < 4) and of B (q < 2), rows 8 g + (l >> 3), lane l fetching the chunk
  // that belongs at LDS position l & 7: logical chunk
  // (l & 7) ^ (4 (g & 1) + (l >> 4)), and g & 1 = w & 1.  And two 4-byte
  // scale loads: into the A stage, waves 0-3 the A-row scales of rows 64 w ..;
  // into the B stage, wave 4 the B scale (lane 0); every other wave and
  // lane reads out of range (zeros into its own unread slot).
  const uint32_t lrow = 8 * w + (lane >> 3);
  const uint32_t lchunk = (lane & 7) ^ (4 * (w & 1) + (lane >> 4));
  const uint32_t a_lane = lrow * lda + 16 * lchunk, b_lane = lrow * ldb + 16 * lchunk;
  // Per-lane offsets of this wave's loads (the slice's k goes in the scalar
  // offset): A row groups q, B row groups i, out of range for rows past M /
  // N; the scale load: waves 0-3 one A row each, wave 4 lane 0 the B scale,
  // everything else out of range.
  uint32_t av[F_A_LD], bv[F_B_LD];
#pragma unroll
  for (int q = 0; q < F_A_LD; ++q)
    av[q] = (int)(lrow + 64 * q) < rows_a ? a_lane + 64 * q * lda : kOutOfRange;
#pragma unroll
  for (int i = 0; i < F_B_LD; ++i)
    bv[i] = (int)(lrow + 64 * i) < rows_b ? b_lane + 64 * i * ldb : kOutOfRange;
  const int sa_row = 64 * w + lane;
  const uint32_t sa_lane =
      w < 4 && sa_row < rows_a ? (uint32_t)sa_row * (uint32_t)a.ssam * 4 : kOutOfRange;
  const uint32_t sb_lane = w == 4 && lane == 0 ? 0u : kOutOfRange;
  // Load q of a batch that fills A stage sa with slice kb_a and B stage sb
  // with slice kb_b: the A-scale load, the A loads, the B loads, the
  // B-scale load.  Chunks past K and slices past the last scale block read
  // zeros.  (q is a compile-time index.)
  auto load_one = [&](int q, int sa, int kb_a, int sb, int kb_b) {
    if (q == 0) {
      // the A-row scales (waves 0-3)
      if constexpr (KIND == kScaleA)
        load_lds4s(rsa, lds32 + a_off(sa) + F_A_BYTES + 256 * w,
                   kb_a < nkb ? sa_lane : kOutOfRange, (uint32_t)(kb_a * a.ssak) * 4);
    } else if (q < F_APART) {
      const uint32_t k0 = (uint32_t)(kb_a * F_BK);
      const bool kin = (int)k0 + 16 * (int)lchunk < K;
      load_lds16s(ra, lds32 + a_off(sa) + (w + 8 * (q - 1)) * 1024, kin ? av[q - 1] : kOutOfRange,
                  k0);
    } else if (q < F_APART + F_B_LD) {
      const int i = q - F_APART;
      const uint32_t k0 = (uint32_t)(kb_b * F_BK);
      const bool kin = (int)k0 + 16 * (int)lchunk < K;
      load_lds16s(rb, lds32 + b_off(sb) + (w + 8 * i) * 1024, kin ? bv[i] : kOutOfRange, k0);
    } else if constexpr (KIND == kScaleB) {
      // the tile's B scale (wave 4)
      load_lds4s(rsb, lds32 + b_off(sb) + F_B_BYTES + 256 * w, kb_b < nkb ? sb_lane : kOutOfRange,
                 (uint32_t)(kb_b * a.ssbk) * 4);
    }
  };

  // Fragment reads: block row r = 16-aligned base + (l & 15); lane group g
  // reads chunks g and g + 4 at positions chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7, g = lane >> 4;
  const int rd0 = (lane & 15) * F_BK + ((g ^ sw) * 16), rd1 = (lane & 15) * F_BK + (((g + 4) ^ sw) * 16);
  const int a_rd = 64 * wm * F_BK, b_rd = 64 * wn * F_BK;
  const int sa_rd = F_A_BYTES + (64 * wm + 4 * g) * 4;   // + 64 * i bytes for block i

  f32x4 acc[F_FM][F_FN];
#pragma unroll
  for (int i = 0; i < F_FM; ++i)
#pragma unroll
    for (int j = 0; j < F_FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // A fragments of two slices; B fragments of one (re-read after last use);
  // the next slice's scales
  i32x8 fa[2][F_FM], fb[F_FN];
  f32x4 sa[F_FM];
  float sb;
  auto rd32 = [&](const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p + rd0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + rd1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_a = [&](int buf, int st, int i) { fa[buf][i] = rd32(lds + a_off(st) + a_rd + i * 16 * F_BK); };
  auto read_b = [&](int st, int j) { fb[j] = rd32(lds + b_off(st) + b_rd + j * 16 * F_BK); };
  auto read_s = [&](int sta, int stb) {
    const char* abase = lds + a_off(sta);
#pragma unroll
    for (int i = 0; i < F_FM; ++i) sa[i] = *reinterpret_cast<const f32x4*>(abase + sa_rd + 64 * i);
    sb = *reinterpret_cast<const float*>(lds + b_off(stb) + F_B_BYTES + 256 * 4);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // One slice (A fragments in buffer cur; B fragments and scales of this
  // slice in fb / sa / sb): MFMA n covers block (i, j) = (n % F_FM, n / F_FM)
  // and the fold-in of MFMA n - F_LAG follows it.  Reads of the next slice
  // (A stage nsa, B stage nsb): B fragment j after its last use here, A
  // fragments into buffer cur ^ 1 and the scales spread over the slice; the
  // batch of loads (A(kb_a) -> A stage ld_sa, B(kb_b) -> B stage ld_sb) is
  // spread over the MFMAs.
  auto slice = [&](int cur, int nsa, int nsb, int ld_sa, int kb_a, int ld_sb, int kb_b) {
    f32x4 p[F_LAG + 1];
    float s[F_FM][4];
#pragma unroll
    for (int i = 0; i < F_FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[i][v] = sa[i][v] * sb;
#pragma unroll
    for (int n = 0; n < F_NMMA + F_LAG; ++n) {
      if (n < F_NMMA) {
        const int i = n % F_FM, j = n / F_FM;
        p[n % (F_LAG + 1)] = mfma16x16x128_e4m3(fa[cur][i], fb[j], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        if (i == F_FM - 1) read_b(nsb, j);
      }
      if (n >= F_LAG) {
        const int m = n - F_LAG, i = m % F_FM, j = m / F_FM;
        const f32x4 pm = p[m % (F_LAG + 1)];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] += s[i][v] * pm[v];
      }
      if (n == 1 || n == 5 || n == 9 || n == 13) read_a(cur ^ 1, nsa, n / 4);
      if (n == 10) read_s(nsa, nsb);
#pragma unroll
      for (int q = 0; q < F_NLD; ++q)
        if (q * F_NMMA / F_NLD == n) load_one(q, ld_sa, kb_a, ld_sb, kb_b);
      fence();
    }
  };

  // Pipeline over 128-wide slices kb (A stage kb % AS, B stage kb % BS).
  // Slice kb's batch loads A(kb + AS) into A stage kb % AS and B(kb + BS)
  // into B stage kb % BS: slice kb's own fragments and scales were read
  // during slice kb - 1, so at the barrier that opens slice kb nobody reads
  // those stages any more.  At the start of slice kb, slice kb + 1 must have
  // landed: A(kb + 1) heads batch kb + 1 - AS, and B(kb + 1) is in the same
  // batch (after it) when BS == AS, else in an older one; what may stay in
  // flight is what this wave issued after it: the B part of that batch when
  // B is deeper, and the batches kb + 2 - AS .. kb - 1.  The prologue issues the
  // batches before slice 0 (kb = -BS .. -1, the parts with a slice >= 0) the
  // same way, then waits for slice 0 and reads it.  Slices at or past K load
  // out of range (zeros, no traffic).  A fragment buffers alternate per
  // slice: two slices per trip (a slice past K adds zeros).
#pragma unroll
  for (int j = -BS; j < 0; ++j) {
#pragma unroll
    for (int q = 0; q < F_NLD; ++q)
      if (q < F_APART ? j + AS >= 0 : j + BS >= 0)
        load_one(q, j + AS >= 0 ? j + AS : 0, j + AS, j + BS >= 0 ? j + BS : 0, j + BS);
  }
  // This wave's loads per slice: the code loads and its kind's scale load;
  // at a slice's wait, the loads after A(kb + 1)'s part may stay in flight:
  // the B part of its batch (when B is deeper) and AS - 2 full batches
  // (before slice 0: one batch more).
  constexpr int NLD = F_A_LD + F_B_LD + (KIND == kScaleNone ? 0 : 1);
  constexpr int BPART = F_B_LD + (KIND == kScaleB ? 1 : 0);
  constexpr int B_TAIL = BS > AS ? BPART : 0;
  constexpr int INIT_WAIT = B_TAIL + (AS - 1) * NLD, LOOP_WAIT = B_TAIL + (AS - 2) * NLD;
  static_assert(INIT_WAIT <= 63, "loads in flight must fit the vmcnt counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INIT_WAIT) : "memory");
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < F_FM; ++i) read_a(0, 0, i);
#pragma unroll
  for (int j = 0; j < F_FN; ++j) read_b(0, j);
  read_s(0, 0);
  int sta = 0, stb = 0;  // stages of slice kb
  for (int kb = 0; kb < nkb; kb += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kb + h;
      const int nsa = sta + 1 == AS ? 0 : sta + 1, nsb = stb + 1 == BS ? 0 : stb + 1;
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(LOOP_WAIT, 0));
      asm volatile("s_barrier" ::: "memory");
      fence();
      slice(h, nsa, nsb, sta, k + AS, stb, k + BS);
      sta = nsa;
      stb = nsb;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: lane l holds column l & 15, rows 4 (l >> 4) + v of each block.
  __bf16* C = static_cast<__bf16*>(a.C);
  const int64_t row0 = m0 + 64 * wm + 4 * g, col0 = n0 + 64 * wn + (lane & 15);
#pragma unroll
  for (int i = 0; i < F_FM; ++i)
#pragma unroll
    for (int j = 0; j < F_FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + 16 * i + v, col = col0 + 16 * j;
        if (row < a.M && col < a.N) C[row * a.scm + col] = to_out<__bf16>(acc[i][j][v]);
      }
}

// The tile with each wave in its kind's copy of the K loop (the branch is
// wave-uniform; every copy passes the same barriers).
__device__ __forceinline__ void fp8_tile_waves(const GemmArgs& a, int tm, int tn) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < 4)
    fp8_tile_body<F_AS, F_BS, kScaleA>(a, tm, tn);
  else if (w == 4)
    fp8_tile_body<F_AS, F_BS, kScaleB>(a, tm, tn);
  else
    fp8_tile_body<F_AS, F_BS, kScaleNone>(a, tm, tn);
}

__global__ __launch_bounds__(64 * F_WAVES) void gemm_fp8_tile(GemmArgs a, int tiles_m,
                                                                int tiles_n) {
  int tm, tn;
  tile::tile_coords(tiles_m, tiles_n, 4, tm, tn);
  fp8_tile_waves(a, tm, tn);
}

// Grouped products (see gemm_grouped.hip): the tile's group re-bases A and
// its row scales, B_g and its block scales, and C.
__global__ __launch_bounds__(64 * F_WAVES) void gemm_fp8_grouped(GemmArgs a, GroupTable gt) {
  int g, tm, tn;
  tile::group_coords(gt, F_BM, 4, g, tm, tn);
  GemmArgs ag = a;
  ag.M = gt.row0[g + 1] - gt.row0[g];
  ag.A = static_cast<const uint8_t*>(a.A) + gt.row0[g] * a.sam;
  ag.SA = a.SA + gt.row0[g] * a.ssam;
  ag.B = static_cast<const uint8_t*>(a.B) + g * gt.sbg;
  ag.SB = a.SB + g * gt.ssbg;
  ag.C = static_cast<__bf16*>(a.C) + gt.row0[g] * a.scm;
  fp8_tile_waves(ag, tm, tn);
}

// ---------------------------------------------------------------------------
// Ping-pong form with 256 x 256 tiles.  A 256 x 128 tile moves 48 KiB per
// 128-wide slice for 2 x 256 x 128 x 128 FLOP; a 256 x 256 tile 64 KiB for
// twice the FLOP, i.e. a third fewer bytes per FLOP through each CU's load
// path.  The fp32 accumulators of a 64 x 128 wave tile take 128 VGPRs, so the
// work of each SIMD is split between two waves that take turns, as in the
// ping-pong form of the 16-bit kernel:
//  - waves 0-3 (group 0) own columns 0-127 of the tile, waves 4-7 (group 1)
//    columns 128-255, so each group's columns are exactly one 128-wide B
//    scale block; wave q of a group owns rows 64q .. 64q + 63;
//  - the MFMA runs transposed, P^T = B_blk * A_blk^T, so that lane l's four
//    accumulators of a block belong to one row of C (16 i + l % 16) and four
//    consecutive columns: the fold-in acc += (SA[row] * SB) * P then needs one
//    scale per lane and row block (4 per slice) instead of 16;
//  - intervals separated by workgroup barriers: in each interval one group
//    multiplies a slice (32 MFMAs and the fold-ins, reading the B fragments
//    of its columns from LDS one 16-column block at a time, two blocks ahead)
//    while the other reads the next slice's A fragments, row scales and first
//    two B blocks into registers and issues its loads;
//  - LDS: a ring of two A stages (256 rows x 128 bytes, then the slice's 256
//    A-row scales and the tile's two B scales), loaded by group 0, and one
//    ring per group of its 128 B rows (16 KiB a stage), B0_ST stages loaded
//    by group 0 and B1_ST by group 1.  A group's B rows are read by that
//    group alone, so their stage is free as soon as its own multiply ends,
//    which gives each B load more time in flight than a ring shared by both
//    groups.
// Interval t follows barrier t.  Group 0 reads slice j (A, scales, its first
// B blocks) in interval 2j and multiplies it in 2j + 1; group 1 reads it in
// 2j + 1 and multiplies it in 2j + 2.  So:
//  - A stage j % 2 is free after barrier 2j + 2: group 0 refills it with
//    slice j + 2 in interval 2j + 2 and waits for it before barrier 2j + 4;
//  - group 0's B stage of slice j is free after barrier 2j + 2: group 0
//    refills it with slice j + B0_ST in interval 2j + 2, needed before
//    barrier 2 (j + B0_ST);
//  - group 1's B stage of slice j is free after barrier 2j + 3: group 1
//    refills it with slice j + B1_ST in interval 2j + 3, needed before
//    barrier 2 (j + B1_ST) + 1.
// Each group passes 2 nk + 2 barriers (group 0's last one waits for group 1's
// last multiply: with no conditional barrier in either loop, each loop body
// is one basic block, and the compiler cannot sink the MFMAs of a multiply
// past the barrier that ends it).
constexpr int Q_BM = 256, Q_BN = 256, Q_BK = 128;
constexpr int Q_ROW = 128;                            // bytes of k per staged row
constexpr int Q_A_BYTES = Q_BM * Q_ROW;               // 32 KiB
constexpr int Q_H_BYTES = Q_BN / 2 * Q_ROW;           // one group's B rows: 16 KiB
constexpr int Q_SA = Q_A_BYTES;                       // A-row scales of the slice
constexpr int Q_SB = Q_A_BYTES + 1024;                // the tile's two B scales
constexpr int Q_ASTAGE = Q_A_BYTES + 1024 + 256;
constexpr int Q_A_LOADS = Q_A_BYTES / 1024 / 4;       // 1 KiB loads per wave per slice
constexpr int Q_B_LOADS = Q_H_BYTES / 1024 / 4;
constexpr int Q_FM = 4, Q_FN = 8;                     // 16 x 16 blocks of a wave tile
constexpr int Q_LAG = 3;                              // MFMAs between a block and its fold-in
constexpr int Q_NB = 3;                               // B fragment buffers
constexpr int Q_B0_ST = 3, Q_B1_ST = 2;
static_assert(Q_ASTAGE % 256 == 0, "stage bases on whole bank rows");

template <int B0_ST, int B1_ST>
struct QLds {
  static constexpr int B0 = 2 * Q_ASTAGE;                   // group 0's B ring
  static constexpr int B1 = B0 + B0_ST * Q_H_BYTES;         // group 1's B ring
  static constexpr int BYTES = B1 + B1_ST * Q_H_BYTES;
  static_assert(BYTES <= 160 * 1024, "stages must fit the LDS");
};

__device__ __forceinline__ void load_lds4(const i32x4& desc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(desc) : "memory");
}

template <int B0_ST = Q_B0_ST, int B1_ST = Q_B1_ST>
__device__ __forceinline__ void fp8_pp_body(const GemmArgs& a, int tm, int tn) {
  static_assert(B0_ST >= 2 && B1_ST >= 2, "at least two stages per B ring");
  typedef QLds<B0_ST, B1_ST> L;
  char* const lds = fp8_lds<L::BYTES>();
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
  auto a_off = [](int st) { return st * Q_ASTAGE; };

  const int64_t m0 = (int64_t)tm * Q_BM, n0 = (int64_t)tn * Q_BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = w >> 2, q = w & 3;  // group, wave within the group (its SIMD)
  const int K = (int)a.K;
  const int nkb = (K + Q_BK - 1) / Q_BK;
  // Slice order as in the bf16 eight-wave kernel: workgroups of odd dispatch
  // rounds take the K blocks from the top down, starting with the rows the
  // round before read last (still in the last-level cache).  slice_kb(j) is
  // the K block of the j-th slice taken; past the end it is -1 (zeros).
  const bool down = (blockIdx.x / tile::kRoundWgs) & 1;
  auto slice_kb = [&](int j) { return j >= nkb ? -1 : (down ? nkb - 1 - j : j); };
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  // this group's B ring
  const int b_ring = g == 0 ? L::B0 : L::B1;
  auto b_off = [&](int st) { return b_ring + st * Q_H_BYTES; };

  // Code tiles as descriptors ending at the last valid row (A rows m0 ..,
  // this group's B rows n0 + 128 g ..); the tile's scales: A rows m0 ..
  // (SA[i, kb] at i * ssam + kb * ssak floats) and B scale rows n0 / 128 and
  // n0 / 128 + 1 (the second only if N reaches it).
  const int rows_a = (int)min<int64_t>(Q_BM, a.M - m0);
  const int rows_b = (int)max<int64_t>(0, min<int64_t>(Q_BN / 2, a.N - n0 - 128 * g));
  const uint8_t* Ab = static_cast<const uint8_t*>(a.A) + m0 * a.sam;
  const uint8_t* Bb = static_cast<const uint8_t*>(a.B) + (n0 + 128 * g) * a.sbn;
  const i32x4 ra = make_desc(Ab, (uint32_t)((rows_a - 1) * lda + K));
  const i32x4 rb = make_desc(Bb, rows_b > 0 ? (uint32_t)((rows_b - 1) * ldb + K) : 0u);
  const int nsb = (int)min<int64_t>(2, cdiv(a.N, 128) - n0 / 128);
  const float* SAb = a.SA + m0 * a.ssam;
  const float* SBb = a.SB + (n0 / 128) * a.ssbn;
  const i32x4 rsa = make_desc(SAb, (uint32_t)(((rows_a - 1) * a.ssam + (nkb - 1) * a.ssak + 1) * 4));
  const i32x4 rsb = make_desc(SBb, (uint32_t)(((nsb - 1) * a.ssbn + (nkb - 1) * a.ssbk + 1) * 4));

  // Code loads: wave q's i-th load of a stage fills rows 32 i + 8 q .. + 7;
  // lane l writes row 32 i + 8 q + (l >> 3) at chunk position l & 7, i.e.
  // logical chunk (l & 7) ^ (4 (q & 1) + (l >> 4)) (swizzle c ^ ((r >> 1) & 7)).
  // Rows past the last valid row fall outside the descriptor (zeros).
  const uint32_t lrow = 8 * q + (lane >> 3);
  const uint32_t lchunk = (lane & 7) ^ (4 * (q & 1) + (lane >> 4));
  auto load_rows = [&](const i32x4& desc, uint32_t ld, uint32_t base, int kb, auto n_loads) {
    const int k0 = kb * Q_BK;
    const bool kin = kb >= 0 && k0 + 16 * (int)lchunk < K;
    const uint32_t lane_off = lrow * ld + 16 * lchunk + (uint32_t)k0;
#pragma unroll
    for (int i = 0; i < decltype(n_loads)::value; ++i)
      load_lds16(desc, base + i * 4096, kin ? lane_off + i * 32 * ld : kOutOfRange);
  };
  typedef std::integral_constant<int, Q_A_LOADS> NA;
  typedef std::integral_constant<int, Q_B_LOADS> NB;
  auto load_a = [&](int st, int kb) { load_rows(ra, lda, lds32 + a_off(st) + q * 1024, kb, NA()); };
  auto load_b = [&](int st, int kb) { load_rows(rb, ldb, lds32 + b_off(st) + q * 1024, kb, NB()); };
  // Scale loads (group 0): wave q the A-row scales of rows 64 q + l, wave 0
  // lanes 0-1 also the two B scales; everything else reads zeros.
  const int sa_row = 64 * q + lane;
  const bool sa_in = sa_row < rows_a, sb_in = lane < nsb;
  const uint32_t sa_lane = (uint32_t)sa_row * (uint32_t)a.ssam * 4;
  const uint32_t sb_lane = (uint32_t)lane * (uint32_t)a.ssbn * 4;
  auto load_scales = [&](int st, int kb) {
    const bool kin = kb >= 0 && kb < nkb;
    load_lds4(rsa, lds32 + a_off(st) + Q_SA + 256 * q,
              kin && sa_in ? sa_lane + (uint32_t)(kb * a.ssak) * 4 : kOutOfRange);
    if (q == 0)
      load_lds4(rsb, lds32 + a_off(st) + Q_SB,
                kin && sb_in ? sb_lane + (uint32_t)(kb * a.ssbk) * 4 : kOutOfRange);
  };

  // Fragment reads (16x16x128): block row (16-aligned base) + (l & 15);
  // lane group u = l >> 4 reads chunks u and u + 4 of the 128-byte row, at
  // positions chunk ^ ((l >> 1) & 7).  A and B take the same k assignment.
  const int sw = (lane >> 1) & 7, u = lane >> 4;
  const int rd0 = (lane & 15) * Q_ROW + ((u ^ sw) * 16);
  const int rd1 = (lane & 15) * Q_ROW + (((u + 4) ^ sw) * 16);
  auto rd32 = [&](const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p + rd0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + rd1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  const int a_rd = 64 * q * Q_ROW;
  const int s_rd = Q_SA + (64 * q + (lane & 15)) * 4;

  // acc[j][i]: block of tile columns 16 j .. (this group's) and rows 16 i ..
  // (this wave's); lane l holds row 16 i + (l & 15), columns 16 j + 4 (l >> 4) + v.
  f32x4 acc[Q_FN][Q_FM];
#pragma unroll
  for (int j = 0; j < Q_FN; ++j)
#pragma unroll
    for (int i = 0; i < Q_FM; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  i32x8 fa[Q_FM], fb[Q_NB];
  float s[Q_FM];  // SA[row] * SB of this lane's rows for the slice
  auto read_b = [&](int st, int j) { return rd32(lds + b_off(st) + j * 16 * Q_ROW); };
  // A fragments, scales and the first two B blocks of a slice
  auto read_slice = [&](int sta, int stb) {
    const char* base = lds + a_off(sta);
#pragma unroll
    for (int i = 0; i < Q_FM; ++i) fa[i] = rd32(base + a_rd + i * 16 * Q_ROW);
    const float sb = *reinterpret_cast<const float*>(base + Q_SB + 4 * g);
#pragma unroll
    for (int i = 0; i < Q_FM; ++i)
      s[i] = *reinterpret_cast<const float*>(base + s_rd + 64 * i) * sb;
    fb[0] = read_b(stb, 0);
    fb[1] = read_b(stb, 1);
  };
  // Step boundary of the multiply: the empty asm with a memory clobber keeps
  // the LDS reads where they are written (a scheduling fence alone lets
  // instruction selection hoist all of them to the top, which needs 40 more
  // VGPRs), the scheduling fence keeps MFMAs and fold-ins in their steps.
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // One slice from B stage st: MFMA n covers block (j, i) = (n / 4, n % 4)
  // and the fold-in of MFMA n - Q_LAG follows it; the fragments of column
  // block j + 2 are read when block j's first MFMA has been issued.
  auto multiply = [&](int st) {
    f32x4 p[Q_LAG + 1];
#pragma unroll
    for (int n = 0; n < Q_FN * Q_FM + Q_LAG; ++n) {
      if (n < Q_FN * Q_FM) {
        const int j = n / Q_FM, i = n % Q_FM;
        p[n % (Q_LAG + 1)] = mfma16x16x128_e4m3(fb[j % Q_NB], fa[i], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        if (i == 0 && j + 2 < Q_FN) fb[(j + 2) % Q_NB] = read_b(st, j + 2);
      }
      if (n >= Q_LAG) {
        const int m = n - Q_LAG, j = m / Q_FM, i = m % Q_FM;
        const f32x4 pm = p[m % (Q_LAG + 1)];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[j][i][v] += s[i] * pm[v];
      }
      fence();
    }
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_lds = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // wait until at most N of this wave's loads are in flight
  auto wait_loads = [](auto n) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(n)::value) : "memory");
  };

  if (g == 0) {
    // Per iteration j: A(j + 1) with its scales, then B0(j + B0_ST - 1).
    // Before barrier 2j + 2, A(j + 1) and B0(j + 1) must have landed: B0(j +
    // 1) was issued B0_ST - 2 iterations back, so the B0 loads of the last
    // B0_ST - 2 iterations may stay in flight (scale loads precede them).
    load_a(0, slice_kb(0));
    load_scales(0, slice_kb(0));
#pragma unroll
    for (int x = 0; x < B0_ST - 1; ++x) load_b(x, slice_kb(x));
    wait_loads(std::integral_constant<int, (B0_ST - 2) * Q_B_LOADS>());
    barrier();                                   // 0
    int sta = 0, stb = 0;
    for (int j = 0; j < nkb; ++j) {
      const int nsta = sta ^ 1, lstb = stb == 0 ? B0_ST - 1 : stb - 1;
      load_a(nsta, slice_kb(j + 1));             // into slice j - 1's stage
      load_scales(nsta, slice_kb(j + 1));
      load_b(lstb, slice_kb(j + B0_ST - 1));     // into slice j - 1's stage
      read_slice(sta, stb);
      wait_lds();
      barrier();                                 // 2j + 1
      multiply(stb);
      wait_loads(std::integral_constant<int, (B0_ST - 2) * Q_B_LOADS>());
      barrier();                                 // 2j + 2
      sta = nsta;
      stb = stb + 1 == B0_ST ? 0 : stb + 1;
    }
    barrier();                                   // 2 nk + 1: group 1's last multiply
  } else {
    // Per iteration j: B1(j + B1_ST - 1).  Before barrier 2j + 3, B1(j + 1)
    // must have landed: issued B1_ST - 2 iterations back.
#pragma unroll
    for (int x = 0; x < B1_ST - 1; ++x) load_b(x, slice_kb(x));
    wait_loads(std::integral_constant<int, (B1_ST - 2) * Q_B_LOADS>());
    barrier();                                   // 0
    barrier();                                   // 1
    int sta = 0, stb = 0;
    for (int j = 0; j < nkb; ++j) {
      const int lstb = stb == 0 ? B1_ST - 1 : stb - 1;
      load_b(lstb, slice_kb(j + B1_ST - 1));     // into slice j - 1's stage
      read_slice(sta, stb);
      wait_lds();
      barrier();                                 // 2j + 2
      multiply(stb);
      wait_loads(std::integral_constant<int, (B1_ST - 2) * Q_B_LOADS>());
      barrier();                                 // 2j + 3
      sta ^= 1;
      stb = stb + 1 == B1_ST ? 0 : stb + 1;
    }
  }
  // loads past the last slice (zeros) land before the LDS is released
  wait_loads(std::integral_constant<int, 0>());

  // Epilogue: round each accumulator to bf16 and store it inside M x N.
  __bf16* C = static_cast<__bf16*>(a.C);
  const int64_t row0 = m0 + 64 * q + (lane & 15);
  const int64_t col0 = n0 + 128 * g + 4 * u;
  const bool whole = m0 + Q_BM <= a.M && n0 + Q_BN <= a.N && a.scm % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(a.C) & 7) == 0;
  if (whole) {
#pragma unroll
    for (int j = 0; j < Q_FN; ++j)
#pragma unroll
      for (int i = 0; i < Q_FM; ++i) {
        const bf16x4 o = {to_out<__bf16>(acc[j][i][0]), to_out<__bf16>(acc[j][i][1]),
                          to_out<__bf16>(acc[j][i][2]), to_out<__bf16>(acc[j][i][3])};
        *reinterpret_cast<bf16x4*>(C + (row0 + 16 * i) * a.scm + col0 + 16 * j) = o;
      }
  } else {
#pragma unroll
    for (int j = 0; j < Q_FN; ++j)
#pragma unroll
      for (int i = 0; i < Q_FM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = row0 + 16 * i, col = col0 + 16 * j + v;
          if (row < a.M && col < a.N) C[row * a.scm + col] = to_out<__bf16>(acc[j][i][v]);
        }
  }
}

__global__ __launch_bounds__(512) void gemm_fp8_pp(GemmArgs a, int tiles_m, int tiles_n) {
  int tm, tn;
  tile::tile_coords(tiles_m, tiles_n, 4, tm, tn);
  fp8_pp_body(a, tm, tn);
}

__global__ __launch_bounds__(512) void gemm_fp8_grouped_pp(GemmArgs a, GroupTable gt) {
  int g, tm, tn;
  tile::group_coords(gt, Q_BM, 4, g, tm, tn);
  GemmArgs ag = a;
  ag.M = gt.row0[g + 1] - gt.row0[g];
  ag.A = static_cast<const uint8_t*>(a.A) + gt.row0[g] * a.sam;
  ag.SA = a.SA + gt.row0[g] * a.ssam;
  ag.B = static_cast<const uint8_t*>(a.B) + g * gt.sbg;
  ag.SB = a.SB + g * gt.ssbg;
  ag.C = static_cast<__bf16*>(a.C) + gt.row0[g] * a.scm;
  fp8_pp_body(ag, tm, tn);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Both code operands K-contiguous with 16-byte aligned rows, K a multiple of
// 16 (whole 16-byte chunks); descriptor ranges fit 31 bits.
bool accepts(Op op, const GemmArgs& a) {
  if (op != Op::FP8) return false;
  if (a.K == 0 || a.K % 16 != 0) return false;
  if (a.sak != 1 || a.sbk != 1) return false;
  if (a.sam % 16 != 0 || a.sbn % 16 != 0) return false;
  if (!aligned16(a.A) || !aligned16(a.B)) return false;
  if ((reinterpret_cast<uintptr_t>(a.SA) & 3) || (reinterpret_cast<uintptr_t>(a.SB) & 3)) return false;
  const int64_t lim = int64_t(1) << 30, nkb = cdiv(a.K, 128);
  if (F_BM * a.sam + a.K >= lim || Q_BN * a.sbn + a.K >= lim) return false;
  if ((F_BM * a.ssam + nkb * a.ssak) * 4 >= lim || (a.ssbn + nkb * a.ssbk) * 4 >= lim)
    return false;
  if (a.M > (int64_t(1) << 24) || a.N > (int64_t(1) << 24)) return false;
  return true;
}

// Tile shape of a call: 256 x 256 (ping-pong) unless 256 x 128 tiles finish
// in less time.  Both forms are bound by the bytes each CU moves per slice,
// 64 KiB against 48 KiB, so a tile round of 256 x 256 costs 4 units and one
// of 256 x 128 costs 3 (one tile round: one tile per CU).
constexpr int kCus = 256;
bool wide_tiles(int64_t tiles_m, int64_t N) {
  const int64_t rounds_w = cdiv(tiles_m * cdiv(N, Q_BN), kCus);
  const int64_t rounds_n = cdiv(tiles_m * cdiv(N, F_BN), kCus);
  return 4 * rounds_w <= 3 * rounds_n;
}

hipError_t launch(Op, const GemmArgs& a, const Scratch&, hipStream_t s) {
  if (wide_tiles(cdiv(a.M, 256), a.N)) {
    const int tm = (int)cdiv(a.M, Q_BM), tn = (int)cdiv(a.N, Q_BN);
    hipLaunchKernelGGL(gemm_fp8_pp, dim3(tm * tn), dim3(512), 0, s, a, tm, tn);
  } else {
    const int tm = (int)cdiv(a.M, F_BM), tn = (int)cdiv(a.N, F_BN);
    hipLaunchKernelGGL(gemm_fp8_tile, dim3(tm * tn), dim3(64 * F_WAVES), 0, s, a, tm, tn);
  }
  return hipGetLastError();
}

const char* plan_name(const GemmArgs& a, const Scratch&) {
  return wide_tiles(cdiv(a.M, 256), a.N) ? "tile_fp8_256x256" : "tile_fp8_256x128";
}

struct Grouped8 {
  int64_t G;
  const int64_t* off;
  int64_t N, K;
  const void* A;
  int64_t lda;
  const float* SA;
  int64_t ssam, ssak;
  const void* B;
  int64_t ldb, sbg;
  const float* SB;
  int64_t ssbn, ssbk, ssbg;
  void* C;
  int64_t ldc;
};

// Largest element offset base + sum (n_i - 1) * stride_i + last, checked for
// overflow and kept below 2^60 (byte addresses of fp32 scales included).
bool extent_ok(std::initializer_list<std::pair<int64_t, int64_t>> dims, int64_t last) {
  int64_t e = last, t;
  for (auto d : dims) {
    if (d.first <= 0) continue;
    if (__builtin_mul_overflow(d.first - 1, d.second, &t) || __builtin_add_overflow(e, t, &e))
      return false;
  }
  return e < (int64_t(1) << 60);
}

tg_status validate_grouped(const Grouped8& c) {
  if (c.G < 0 || c.N < 0 || c.K < 0 || c.lda < 0 || c.ssam < 0 || c.ssak < 0 || c.ldb < 0 ||
      c.sbg < 0 || c.ssbn < 0 || c.ssbk < 0 || c.ssbg < 0 || c.ldc < 0)
    return TG_ERR_INVALID_VALUE;
  if (c.G == 0) return TG_SUCCESS;
  if (c.off == nullptr || c.off[0] < 0) return TG_ERR_INVALID_VALUE;
  for (int64_t g = 0; g < c.G; ++g)
    if (c.off[g + 1] < c.off[g]) return TG_ERR_INVALID_VALUE;
  const int64_t rows = c.off[c.G];
  if (rows == 0 || c.N == 0) return TG_SUCCESS;
  if (c.C == nullptr) return TG_ERR_INVALID_VALUE;
  if (c.K > 0 && (c.A == nullptr || c.B == nullptr || c.SA == nullptr || c.SB == nullptr))
    return TG_ERR_INVALID_VALUE;
  if ((rows > 1 && (c.lda < c.K || c.ldc < c.N)) || (c.N > 1 && c.ldb < c.K))
    return TG_ERR_INVALID_VALUE;
  const int64_t nkb = cdiv(c.K, 128), nnb = cdiv(c.N, 128);
  if (!extent_ok({{rows, c.lda}}, c.K) || !extent_ok({{rows, c.ldc}}, c.N) ||
      !extent_ok({{c.G, c.sbg}, {c.N, c.ldb}}, c.K) ||
      !extent_ok({{rows, c.ssam}, {nkb, c.ssak}}, 1) ||
      !extent_ok({{c.G, c.ssbg}, {nnb, c.ssbn}, {nkb, c.ssbk}}, 1) || rows >= (int64_t(1) << 60))
    return TG_ERR_INVALID_VALUE;
  return TG_SUCCESS;
}

// One launch when every group's call would take the tile kernel: at most
// kMaxGroups groups, the single product's conditions, 16-byte aligned group
// bases.
bool grouped_tiled(const Grouped8& c) {
  if (c.G > kMaxGroups || c.K == 0) return false;
  if (c.sbg % 16 != 0) return false;
  for (int64_t g = 0; g < c.G; ++g)
    if (c.off[g + 1] - c.off[g] > (int64_t(1) << 24)) return false;
  GemmArgs a{1, c.N, c.K, c.A, c.lda, 1, c.B, 1, c.ldb, c.SA, c.ssam, c.ssak, c.SB, c.ssbn,
             c.ssbk, c.C, c.ldc};
  return accepts(Op::FP8, a);
}

// Tile shape of a grouped launch (as wide_tiles, over all groups' tile rows).
bool grouped_wide(const Grouped8& c) {
  int64_t tiles_m = 0;
  for (int64_t g = 0; g < c.G; ++g) tiles_m += cdiv(c.off[g + 1] - c.off[g], 256);
  return wide_tiles(tiles_m, c.N);
}

tg_status run_grouped(const Grouped8& c, tg_stream_t stream) {
  tg_status st = validate_grouped(c);
  if (st != TG_SUCCESS || c.G == 0 || c.off[c.G] == c.off[0] || c.N == 0) return st;
  if (grouped_tiled(c)) {
    const bool wide = grouped_wide(c);
    GroupTable gt;
    gt.G = (int)c.G;
    gt.tiles_n = (int)cdiv(c.N, wide ? Q_BN : F_BN);
    gt.sbg = c.sbg;
    gt.ssbg = c.ssbg;
    int64_t tiles = 0;
    for (int64_t g = 0; g <= c.G; ++g) {
      gt.row0[g] = c.off[g] - c.off[0];
      gt.tile0[g] = (int)tiles;
      if (g < c.G) tiles += cdiv(c.off[g + 1] - c.off[g], F_BM) * gt.tiles_n;
    }
    if (tiles >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
    const GemmArgs a{c.off[c.G] - c.off[0], c.N, c.K,
                     static_cast<const uint8_t*>(c.A) + c.off[0] * c.lda, c.lda, 1, c.B, 1, c.ldb,
                     c.SA + c.off[0] * c.ssam, c.ssam, c.ssak, c.SB, c.ssbn, c.ssbk,
                     static_cast<__bf16*>(c.C) + c.off[0] * c.ldc, c.ldc};
    if (wide)
      hipLaunchKernelGGL(gemm_fp8_grouped_pp, dim3((unsigned)tiles), dim3(512), 0,
                         static_cast<hipStream_t>(stream), a, gt);
    else
      hipLaunchKernelGGL(gemm_fp8_grouped, dim3((unsigned)tiles), dim3(64 * F_WAVES), 0,
                         static_cast<hipStream_t>(stream), a, gt);
    return hipGetLastError() == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
  }
  for (int64_t g = 0; g < c.G; ++g) {
    const int64_t m = c.off[g + 1] - c.off[g];
    if (m == 0) continue;
    st = tg_gemm_fp8_blockscaled(m, c.N, c.K, static_cast<const uint8_t*>(c.A) + c.off[g] * c.lda,
                                 c.lda, 1, c.SA + c.off[g] * c.ssam, c.ssam, c.ssak,
                                 static_cast<const uint8_t*>(c.B) + g * c.sbg, 1, c.ldb,
                                 c.SB + g * c.ssbg, c.ssbn, c.ssbk,
                                 static_cast<__bf16*>(c.C) + c.off[g] * c.ldc, c.ldc, 1, stream);
    if (st != TG_SUCCESS) return st;
  }
  return TG_SUCCESS;
}

}  // namespace

const Variant* variant_tile_fp8() {
  static const Variant v = {"tile_fp8", accepts, launch, plan_name, nullptr};
  return &v;
}

}  // namespace tg

extern "C" {

tg_status tg_gemm_grouped_fp8_blockscaled(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                                          const void* A, int64_t lda, const float* SA,
                                          int64_t ssam, int64_t ssak, const void* B, int64_t ldb,
                                          int64_t sbg, const float* SB, int64_t ssbn,
                                          int64_t ssbk, int64_t ssbg, void* C, int64_t ldc,
                                          tg_stream_t stream) {
  return tg::run_grouped(
      tg::Grouped8{G, offsets, N, K, A, lda, SA, ssam, ssak, B, ldb, sbg, SB, ssbn, ssbk, ssbg, C,
                   ldc},
      stream);
}

const char* tg_gemm_grouped_fp8_plan(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                                     const void* A, int64_t lda, const float* SA, int64_t ssam,
                                     int64_t ssak, const void* B, int64_t ldb, int64_t sbg,
                                     const float* SB, int64_t ssbn, int64_t ssbk, int64_t ssbg,
                                     void* C, int64_t ldc) {
  const tg::Grouped8 c{G, offsets, N, K, A, lda, SA, ssam, ssak, B, ldb, sbg, SB, ssbn, ssbk,
                       ssbg, C, ldc};
  if (tg::validate_grouped(c) != TG_SUCCESS) return nullptr;
  if (G == 0 || offsets[G] == offsets[0] || N == 0) return "none";
  if (!tg::grouped_tiled(c)) return "per_group";
  return tg::grouped_wide(c) ? "grouped_tile_fp8_256x256" : "grouped_tile_fp8_256x128";
}

}  // extern "C"
