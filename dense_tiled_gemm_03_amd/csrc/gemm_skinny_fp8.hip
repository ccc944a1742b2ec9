// Skinny block-scaled fp8 product, C = A * B with at most 64 rows (a decode
// step over fp8 weights): A codes M x K with one fp32 scale per 1 x 128 row
// slice, B codes stored N x K with one per 128 x 128 block, bf16 output, as
// tg_gemm_fp8_blockscaled computes it (the block-scaled GEMM of "Getting to
// know TileLang", operator-coverage section; E4M3 FN and amax / 448 scales,
// "TileKernels deep dive" sections 4.3 and 7.2).
//
// B is read exactly once and is nearly all the bytes, so the layout is the
// allocation-free skinny plan of the 16-bit product (gemm_skinny.hip) with
// 128-wide K blocks in place of its 64-wide slices -- a block of fp8 codes is
// the same 128 bytes per row as a 16-bit slice:
//  - each workgroup owns a 32-column strip of C (all rows) over the whole of
//    K, so nothing is combined across workgroups; the strip lies inside one
//    128-column block of B scales;
//  - A and B blocks go through LDS rings of their own (LDS-direct loads; B
//    non-temporal): waves 0-1 load A, wave 0 also the block's A-row scales
//    and wave 1 the strip's B scale (both into the A stage), waves 2-3 load B;
//  - blocks go four to a barrier and wave w multiplies block w of each four
//    (2 MT / 16 16x16x128 MFMAs, transposed as in the fp8 tile kernel so that
//    a lane's accumulators share one A-row scale), folding each block product
//    into its accumulators with that block's SA * SB: the fold-in is linear,
//    so the four waves' partial tiles add up to the product; they are added
//    in wave order through LDS at the end and rounded once to bf16.
// LDS chunk swizzle, descriptors and edges as in the 16-bit kernel: chunk c
// of stage row r at position c ^ ((r >> 1) & 7); rows past M or N and scales
// past the matrices read as zero through the descriptor bounds; blocks past K
// are not loaded, and chunks past K get an out-of-range offset.
#include "../../include/tg_gemm.h"

#include "tile_mfma.hpp"

namespace tg {
namespace {

using tile::kOutOfRange;
using tile::load_lds16;
using tile::load_lds16_nt;
using tile::make_desc;

// Rows of C per workgroup: MT = 16, 32 or 64, the least that holds M.  The
// A stage shrinks with MT and the B ring takes the LDS it frees: a decode
// step with few rows keeps more of B, the stream from HBM, in flight.
constexpr int FN_ = 32;                        // columns of C per workgroup
constexpr int FK = 128;                        // k per block (one scale block)
constexpr int FROW = FK;                       // bytes per stage row
constexpr int FB_BYTES = FN_ * FROW;           // 4 KiB: B stage
constexpr int FA_ST = 12;                      // A ring depth
constexpr int FP = 4;                          // blocks per barrier (one per wave)
constexpr int FB_LD = 2;                       // loads per block of a B wave
constexpr int FRED_PITCH = FN_ + 4;            // fp32 row pitch of the partial tiles
constexpr int F_LDS_MAX = 160 * 1024;

template <int MT>
struct FCfg {
  static constexpr int A_CODES = MT * FROW;             // A codes of a block
  static constexpr int SA = A_CODES;                    // the block's MT A-row scales
  static constexpr int SB = A_CODES + 256;              // the strip's B scale (lane 0 of a load)
  static constexpr int A_BYTES = A_CODES + 512;         // A stage
  static constexpr int A_LD = MT / 16 + 1;              // loads per block of an A wave
  static constexpr int B_ST = (F_LDS_MAX - FA_ST * A_BYTES) / FB_BYTES / FP * FP;
  static constexpr int LDS = FA_ST * A_BYTES + B_ST * FB_BYTES;
  static_assert(MT == 16 || MT == 32 || MT == 64, "16, 32 or 64 rows");
  static_assert(LDS <= F_LDS_MAX, "rings must fit the LDS");
  static_assert(FA_ST % FP == 0 && B_ST % FP == 0 && FA_ST >= 2 * FP && B_ST >= 2 * FP,
                "rings hold whole groups, two groups at least");
  static_assert((FA_ST - FP) * A_LD <= 63 && (B_ST - FP) * FB_LD <= 63,
                "loads in flight must fit the vmcnt counter");
  static_assert(4 * MT * FRED_PITCH * 4 <= LDS, "partial tiles must fit the rings");
  static_assert(A_BYTES % 256 == 0, "stage bases on whole bank rows");
};

// One 4-byte LDS-direct load per lane (the scale loads), issued as the
// 16-byte one is: M0 holds the LDS base, the s_nop covers the M0 hazard.
__device__ __forceinline__ void load_lds4(const i32x4& desc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(desc) : "memory");
}

template <int MT>
__global__ __launch_bounds__(256) void gemm_fp8_skinny(GemmArgs a) {
  typedef FCfg<MT> Cfg;
  constexpr int FA_BYTES = Cfg::A_BYTES, FB_ST = Cfg::B_ST, FA_LD = Cfg::A_LD;
  constexpr int FA_SA = Cfg::SA, FA_SB = Cfg::SB;
  constexpr int NI = MT / 16;                  // 16-row blocks
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS];
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * FN_;
  const int K = (int)a.K;
  const int count = (K + FK - 1) / FK;  // K blocks
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_a = (int)a.M;
  const int rows_b = (int)min<int64_t>(FN_, a.N - n0);
  const uint8_t* Bb = static_cast<const uint8_t*>(a.B) + n0 * a.sbn;
  const i32x4 ra = make_desc(a.A, (uint32_t)((rows_a - 1) * lda + K));
  const i32x4 rb = make_desc(Bb, (uint32_t)((rows_b - 1) * ldb + K));
  const i32x4 rsa = make_desc(
      a.SA, (uint32_t)(((rows_a - 1) * a.ssam + (count - 1) * a.ssak + 1) * 4));
  const i32x4 rsb = make_desc(a.SB + (n0 / 128) * a.ssbn,
                              (uint32_t)(((count - 1) * a.ssbk + 1) * 4));
  const bool loads_a = w < 2;  // wave-uniform

  // Block b's A stage at (b % FA_ST) * FA_BYTES, its B stage after the A
  // ring.  Wave w (0, 1) loads A 8-row groups NI w .. NI w + NI - 1, wave w
  // (2, 3) B groups 2(w - 2) .. + 1; lane l writes group row l >> 3 at chunk
  // position l & 7, i.e. logical chunk (l & 7) ^ (4 (g & 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_a = [&](int blk) {
    if (blk >= count) return;  // nothing past K
    const int k0 = blk * FK;
    const uint32_t stage = lds32 + (blk % FA_ST) * FA_BYTES;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int g = NI * w + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 16 * (int)c < K;
      load_lds16(ra, stage + g * 1024, kin ? (8 * g + lrow) * lda + k0 + 16 * c : kOutOfRange);
    }
    if (w == 0)  // SA[lane, blk]: the A-row scales
      load_lds4(rsa, stage + FA_SA,
                lane < rows_a ? (uint32_t)((lane * a.ssam + blk * a.ssak) * 4) : kOutOfRange);
    else  // SB[n0 / 128, blk] in lane 0
      load_lds4(rsb, stage + FA_SB, lane == 0 ? (uint32_t)(blk * a.ssbk * 4) : kOutOfRange);
  };
  auto load_b = [&](int blk) {
    if (blk >= count) return;
    const int k0 = blk * FK;
    const uint32_t stage = lds32 + FA_ST * FA_BYTES + (blk % FB_ST) * FB_BYTES;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g = 2 * (w - 2) + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 16 * (int)c < K;
      load_lds16_nt(rb, stage + g * 1024, kin ? (8 * g + lrow) * ldb + k0 + 16 * c : kOutOfRange);
    }
  };
  // Waits for this wave's stream, as in the 16-bit kernel: before the first
  // group, blocks 0 .. FP - 1 landed (the ring's other ST - FP may be in
  // flight); before the group after blocks i .. i + FP - 1 is read, blocks
  // .. i + 2 FP - 1 landed (all, near the end of K, where fewer follow).
  auto wait_first = [&]() {
    if (loads_a) {
      if (FA_ST <= count) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((FA_ST - FP) * FA_LD) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (FB_ST <= count) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((FB_ST - FP) * FB_LD) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  auto wait_next = [&](int i) {
    if (loads_a) {
      if (i + FA_ST <= count)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((FA_ST - 2 * FP) * FA_LD) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    } else {
      if (i + FB_ST <= count)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((FB_ST - 2 * FP) * FB_LD) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
  };

  // Wave w's fragments of block i + w (16x16x128): 16-row block base +
  // (l & 15), lane group u = l >> 4 reading chunks u and u + 4 at positions
  // chunk ^ ((l >> 1) & 7); A and B take the same k assignment.  Lane l's
  // accumulators of block (j, i) hold row 16 i + (l & 15), columns
  // 16 j + 4 u + v, so it needs the scales of rows 16 i + (l & 15).
  const int sw = (lane >> 1) & 7, u = lane >> 4;
  const int rd0 = (lane & 15) * FROW + ((u ^ sw) * 16);
  const int rd1 = (lane & 15) * FROW + (((u + 4) ^ sw) * 16);
  auto rd32 = [&](const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p + rd0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + rd1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  f32x4 acc[2][NI];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  i32x8 fa[2][NI], fb[2][2];
  float s[2][NI];
  auto read_block = [&](int buf, int blk) {
    const char* ab = lds + (blk % FA_ST) * FA_BYTES;
    const char* bb = lds + FA_ST * FA_BYTES + (blk % FB_ST) * FB_BYTES;
    const float sb = *reinterpret_cast<const float*>(ab + FA_SB);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      fa[buf][i] = rd32(ab + i * 16 * FROW);
      s[buf][i] = *reinterpret_cast<const float*>(ab + FA_SA + (16 * i + (lane & 15)) * 4) * sb;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[buf][j] = rd32(bb + j * 16 * FROW);
  };
  // The group of blocks i .. i + FP - 1 (this wave's block i + w read into
  // buffer cur): wait for the next group and for every wave's reads of this
  // one, refill this group's slots with the blocks a ring's depth later,
  // read this wave's block of the next group, multiply and fold in this one.
  auto step = [&](int i, int cur) {
    wait_next(i);
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int h = 0; h < FP; ++h) {
      if (loads_a) load_a(i + h + FA_ST);
      else load_b(i + h + FB_ST);
    }
    if (i + FP + w < count) read_block(cur ^ 1, i + FP + w);
    __builtin_amdgcn_sched_barrier(0);
    if (i + w < count) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          const f32x4 p = mfma16x16x128_e4m3(fb[cur][j], fa[cur][ii], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[j][ii][v] += s[cur][ii] * p[v];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if (loads_a) {
#pragma unroll
    for (int p = 0; p < FA_ST; ++p) load_a(p);
  } else {
#pragma unroll
    for (int p = 0; p < FB_ST; ++p) load_b(p);
  }
  wait_first();
  asm volatile("s_barrier" ::: "memory");
  if (w < count) read_block(0, w);
  int i = 0;
  for (; i + FP < count; i += 2 * FP) {
    step(i, 0);
    step(i + FP, 1);
  }
  if (i < count) step(i, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The four waves' partial tiles through LDS (row 16 i + (l & 15), columns
  // 16 j + 4 u .. + 3 of wave w's tile), then thread t, step e: float4
  // q = 256 e + t of the MT x 32 tile (row q >> 3, columns 4 (q & 7) .. + 3),
  // the sum of the four partials in wave order, rounded once to bf16.
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
      *reinterpret_cast<f32x4*>(red + (w * MT + 16 * ii + (lane & 15)) * FRED_PITCH + 16 * j +
                                4 * u) = acc[j][ii];
  __syncthreads();
  __bf16* Cb = static_cast<__bf16*>(a.C);
  const int t = threadIdx.x;
#pragma unroll
  for (int e = 0; e < (MT * FN_ / 4 + 255) / 256; ++e) {
    const int q = 256 * e + t, row = q >> 3, col = 4 * (q & 7);
    if (row >= MT) continue;
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      x += *reinterpret_cast<const f32x4*>(red + (ww * MT + row) * FRED_PITCH + col);
    if (row >= a.M) continue;
    __bf16* C = Cb + (int64_t)row * a.scm + n0 + col;
    bf16x4 o;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) o[jj] = to_out<__bf16>(x[jj]);
    if (n0 + col + 4 <= a.N && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
      *reinterpret_cast<bf16x4*>(C) = o;
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (n0 + col + jj < a.N) C[jj] = o[jj];
    }
  }
}

// The split plan, for a caller that gives a workspace: the strip kernel above
// reads all of A once per 32 columns, which at 64 rows is twice the bytes of
// B it reads, from L2.  Here, as in the 16-bit split plan (gemm_skinny.hip), a
// workgroup owns 128 columns of C over one of `splits` ranges of the K
// blocks, so A is read once per 128 columns and each workgroup moves about
// half the bytes:
//  - one ring of XST stages shared by the 4 waves, one barrier per block;
//    a stage holds the block's 64 A rows, their scales and the strip's B
//    scale, then the strip's 128 B rows; wave w loads A rows 16w .. 16w + 15
//    and B rows 32w .. 32w + 31, wave 0 the A-row scales, wave 1 the B scale;
//  - wave w owns columns 32w .. 32w + 31 of the strip, all 64 rows: per block
//    8 16x16x128 MFMAs, transposed as above, each folded in with SA * SB;
//  - the fp32 64 x 128 partial tile goes to the workspace; the last of a
//    strip's workgroups to finish (a device-scope counter) adds the strip's
//    partial tiles in split order, rounds once to bf16 and clears the counter.
constexpr int XM = 64, XN = 128;               // rows, columns of C per workgroup
constexpr int X_SA = 64 * FROW;                // 8 KiB of A codes, then the A-row scales
constexpr int X_SB = X_SA + 256;               // the strip's B scale
constexpr int X_B = X_SA + 512;                // B codes
constexpr int X_STAGE = X_B + XN * FROW;       // 24.5 KiB
constexpr int XST = 6;                         // ring depth
constexpr int X_NLD = 6;                       // 16-byte loads per wave per block
constexpr int X_PITCH = XN + 4;                // fp32 row pitch of the tile in LDS
constexpr int kMinBlocks = 4;                  // fewest K blocks per split
constexpr int kCus = 256;
constexpr int kCoherent = 0x10;                // sc1: device-coherent buffer access
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
static_assert(XST * X_STAGE <= F_LDS_MAX, "the ring fits the LDS");
static_assert(XM * X_PITCH * 4 <= XST * X_STAGE, "the tile fits the ring");
static_assert(XST * (X_NLD + 1) <= 63, "loads in flight fit the vmcnt counter");
static_assert(X_B % 256 == 0 && X_STAGE % 256 == 0, "stage parts on whole bank rows");

__global__ __launch_bounds__(256) void gemm_fp8_skinny_split(GemmArgs a, int splits, float* part,
                                                             int* counters) {
  __shared__ __attribute__((aligned(1024))) char lds[XST * X_STAGE];
  __shared__ int last;  // this workgroup is the strip's last to finish
  const uint32_t lds32 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x / splits, split = blockIdx.x % splits;
  const int64_t n0 = (int64_t)strip * XN;
  const int K = (int)a.K;
  const int nkb = (K + FK - 1) / FK;
  const int b_begin = (int)((int64_t)split * nkb / splits);
  const int b_end = (int)((int64_t)(split + 1) * nkb / splits);
  const int count = b_end - b_begin;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;
  const int rows_a = (int)a.M;
  const int rows_b = (int)min<int64_t>(XN, a.N - n0);
  const uint8_t* Bb = static_cast<const uint8_t*>(a.B) + n0 * a.sbn;
  const i32x4 ra = make_desc(a.A, (uint32_t)((rows_a - 1) * lda + K));
  const i32x4 rb = make_desc(Bb, (uint32_t)((rows_b - 1) * ldb + K));
  const i32x4 rsa = make_desc(
      a.SA, (uint32_t)(((rows_a - 1) * a.ssam + (nkb - 1) * a.ssak + 1) * 4));
  const i32x4 rsb = make_desc(a.SB + strip * a.ssbn, (uint32_t)(((nkb - 1) * a.ssbk + 1) * 4));
  const bool scales = w < 2;  // waves 0 and 1 load a scale too (wave-uniform)

  // Block blk (blk - b_begin = i) in slot i % XST.  8-row groups: A group g
  // at g KiB, B group g at X_B + g KiB; lane l writes group row l >> 3 at
  // chunk position l & 7, i.e. logical chunk (l & 7) ^ (4 (g & 1) + (l >> 4)).
  const uint32_t lrow = lane >> 3;
  const uint32_t lc0 = (lane & 7) ^ (lane >> 4), lc1 = (lane & 7) ^ (4 + (lane >> 4));
  auto load_block = [&](int slot, int blk) {
    if (blk >= b_end) return;  // nothing past the range
    const int k0 = blk * FK;
    const uint32_t stage = lds32 + slot * X_STAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g = 2 * w + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 16 * (int)c < K;
      load_lds16(ra, stage + g * 1024, kin ? (8 * g + lrow) * lda + k0 + 16 * c : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * w + j;
      const uint32_t c = (g & 1) ? lc1 : lc0;
      const bool kin = k0 + 16 * (int)c < K;
      load_lds16_nt(rb, stage + X_B + g * 1024,
                    kin ? (8 * g + lrow) * ldb + k0 + 16 * c : kOutOfRange);
    }
    if (w == 0)  // SA[lane, blk]
      load_lds4(rsa, stage + X_SA,
                lane < rows_a ? (uint32_t)((lane * a.ssam + blk * a.ssak) * 4) : kOutOfRange);
    else if (w == 1)  // SB[strip, blk] in lane 0
      load_lds4(rsb, stage + X_SB, lane == 0 ? (uint32_t)(blk * a.ssbk * 4) : kOutOfRange);
  };

  // Fragments as in the strip kernel: A row blocks i (rows 16 i + (l & 15)),
  // this wave's B column blocks j (strip rows 32 w + 16 j + (l & 15)).
  const int sw = (lane >> 1) & 7, u = lane >> 4;
  const int rd0 = (lane & 15) * FROW + ((u ^ sw) * 16);
  const int rd1 = (lane & 15) * FROW + (((u + 4) ^ sw) * 16);
  auto rd32 = [&](const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p + rd0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + rd1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  f32x4 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  i32x8 fa[2][4], fb[2][2];
  float s[2][4];
  auto read_block = [&](int buf, int slot) {
    const char* st = lds + slot * X_STAGE;
    const float sb = *reinterpret_cast<const float*>(st + X_SB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[buf][i] = rd32(st + i * 16 * FROW);
      s[buf][i] = *reinterpret_cast<const float*>(st + X_SA + (16 * i + (lane & 15)) * 4) * sb;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[buf][j] = rd32(st + X_B + (32 * w + 16 * j) * FROW);
  };
  // Block i: wait until block i + 1 has landed (at most the loads of the
  // XST - 2 blocks issued after it outstanding; all, near the end of the
  // range) and every wave's reads of block i are done; refill block i's slot
  // with block i + XST; read block i + 1; multiply block i.
  auto step = [&](int i, int cur) {
    if (i + XST - 1 < count) {
      if (scales)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((XST - 2) * (X_NLD + 1)) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((XST - 2) * X_NLD) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    load_block(i % XST, b_begin + i + XST);
    if (i + 1 < count) read_block(cur ^ 1, (i + 1) % XST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const f32x4 p = mfma16x16x128_e4m3(fb[cur][j], fa[cur][ii], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[j][ii][v] += s[cur][ii] * p[v];
      }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int p = 0; p < XST; ++p) load_block(p, b_begin + p);
  if (XST <= count) {
    if (scales)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((XST - 1) * (X_NLD + 1)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((XST - 1) * X_NLD) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_barrier" ::: "memory");
  read_block(0, 0);
  int i = 0;
  for (; i + 1 < count; i += 2) {
    step(i, 0);
    step(i + 1, 1);
  }
  if (i < count) step(i, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The 64 x 128 tile through LDS (wave w's lane l: row 16 i + (l & 15),
  // columns 32 w + 16 j + 4 u .. + 3), then thread t, step e: float4
  // q = 256 e + t (row q >> 5, columns 4 (q & 31) .. + 3).
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      *reinterpret_cast<f32x4*>(red + (16 * ii + (lane & 15)) * X_PITCH + 32 * w + 16 * j +
                                4 * u) = acc[j][ii];
  __syncthreads();
  const int t = threadIdx.x;
  f32x4 x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = 256 * e + t;
    x[e] = *reinterpret_cast<const f32x4*>(red + (q >> 5) * X_PITCH + 4 * (q & 31));
  }
  if (splits > 1) {
    // Publish this split's tile (device-coherent stores, complete before the
    // barrier ahead of the counter increment); the strip's last workgroup
    // adds every split's tile in split order, so the sum does not depend on
    // which finishes last, and clears the counter for the next call.
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        part + (int64_t)strip * splits * XM * XN, (short)0, splits * XM * XN * 4, 0x00020000);
    // only the rows of C are stored and read (row (256 e + t) >> 5 < M)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * e + (t >> 5) < a.M)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[e]), rp,
                                               (split * XM * XN + 4 * (256 * e + t)) * 4, 0,
                                               kCoherent);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0) last = atomicAdd(counters + strip, 1) == splits - 1;
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int sp0 = 0; sp0 < splits; sp0 += 4) {
      u32x4 y[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          y[j][e] = 8 * e + (t >> 5) < a.M && sp0 + j < splits
                        ? __builtin_amdgcn_raw_buffer_load_b128(
                              rp, ((sp0 + j) * XM * XN + 4 * (256 * e + t)) * 4, 0, kCoherent)
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (sp0 + j < splits)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += __builtin_bit_cast(f32x4, y[j][e]);
    }
    if (t == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __bf16* Cb = static_cast<__bf16*>(a.C);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = 256 * e + t, row = q >> 5, col = 4 * (q & 31);
    if (row >= a.M) continue;
    __bf16* C = Cb + (int64_t)row * a.scm + n0 + col;
    bf16x4 o;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) o[jj] = to_out<__bf16>(x[e][jj]);
    if (n0 + col + 4 <= a.N && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
      *reinterpret_cast<bf16x4*>(C) = o;
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (n0 + col + jj < a.N) C[jj] = o[jj];
    }
  }
}

// Splits of the K blocks: about one workgroup per CU, each with at least
// kMinBlocks blocks; 1 (no split plan) where the strip kernel is as fast.
// Both kernels stream the same B bytes per CU; the split saves A bytes and
// fills the CUs when the strip grid does not, but pays a fixed cost for the
// combine of the partial tiles that grows with the splits.  It is taken, as
// measured, for more than 32 rows (with fewer, A is small and the strip
// kernel keeps more of B in flight) when each strip workgroup has a long
// run of K blocks (strip rounds x blocks >= kLongBlocks), or when the strip
// grid fills at most half the CUs and K has at least kHalfGridBlocks blocks.
constexpr int kLongBlocks = 96;
constexpr int kHalfGridBlocks = 56;
int choose_splits(const GemmArgs& a) {
  if (a.M <= 32) return 1;
  const int64_t strips = cdiv(a.N, XN), nkb = cdiv(a.K, FK);
  int64_t sp = kCus / strips;
  if (sp > nkb / kMinBlocks) sp = nkb / kMinBlocks;
  if (sp < 2) return 1;
  const int64_t strip_wgs = cdiv(a.N, FN_);
  const bool long_strips = cdiv(strip_wgs, kCus) * nkb >= kLongBlocks;
  const bool half_grid = strip_wgs <= kCus / 2 && nkb >= kHalfGridBlocks;
  return long_strips || half_grid ? (int)sp : 1;
}

// The split plan's scratch: a counter per strip in the fixed counter area,
// then each split's 64 x 128 fp32 tile (0: no split plan for this call, or
// a B strip whose offsets leave the descriptor range).
size_t scratch_bytes(const GemmArgs& a) {
  const int64_t strips = cdiv(a.N, XN);
  const int splits = choose_splits(a);
  if (splits == 1 || strips > kWorkspaceCounters) return 0;
  if (XN * a.sbn + a.K >= (int64_t(1) << 30)) return 0;
  return kWorkspaceCounterBytes + (size_t)strips * splits * XM * XN * 4;
}

bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// At most 64 rows, both code matrices K-contiguous with 16-byte aligned rows
// and K a multiple of 16 (whole 16-byte chunks); 4-byte aligned scales;
// offsets inside the descriptors' 31-bit ranges.
bool accepts(Op op, const GemmArgs& a) {
  if (op != Op::FP8) return false;
  if (a.M > 64 || a.K == 0 || a.K % 16 != 0) return false;
  if (a.sak != 1 || a.sbk != 1) return false;
  if (a.sam % 16 != 0 || a.sbn % 16 != 0) return false;
  if (!aligned16p(a.A) || !aligned16p(a.B)) return false;
  if ((reinterpret_cast<uintptr_t>(a.SA) & 3) || (reinterpret_cast<uintptr_t>(a.SB) & 3)) return false;
  const int64_t lim = int64_t(1) << 30, nkb = cdiv(a.K, FK);
  if (64 * a.sam + a.K >= lim || FN_ * a.sbn + a.K >= lim) return false;
  if ((64 * a.ssam + nkb * a.ssak) * 4 >= lim || (nkb * a.ssbk + 1) * 4 >= lim) return false;
  if (a.N > (int64_t(1) << 30)) return false;
  return true;
}

hipError_t launch(Op, const GemmArgs& a, const Scratch& ws, hipStream_t s) {
  if (scratch_fits(ws, scratch_bytes(a))) {
    const int splits = choose_splits(a);
    const dim3 grid((unsigned)(cdiv(a.N, XN) * splits));
    hipLaunchKernelGGL(gemm_fp8_skinny_split, grid, dim3(256), 0, s, a, splits,
                       reinterpret_cast<float*>(ws.ptr + kWorkspaceCounterBytes),
                       reinterpret_cast<int*>(ws.ptr));
    return hipGetLastError();
  }
  const dim3 grid((unsigned)cdiv(a.N, FN_));
  if (a.M <= 16)
    hipLaunchKernelGGL(gemm_fp8_skinny<16>, grid, dim3(256), 0, s, a);
  else if (a.M <= 32)
    hipLaunchKernelGGL(gemm_fp8_skinny<32>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_fp8_skinny<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

const char* const kSplitNames[] = {
    "skinny_fp8_64x32",          "skinny_fp8_64x32",          "skinny_fp8_64x128_splitk2",
    "skinny_fp8_64x128_splitk3", "skinny_fp8_64x128_splitk4", "skinny_fp8_64x128_splitk5",
    "skinny_fp8_64x128_splitk6", "skinny_fp8_64x128_splitk7", "skinny_fp8_64x128_splitk8"};
const char* name_of(const GemmArgs& a, const Scratch& ws) {
  if (!scratch_fits(ws, scratch_bytes(a))) return "skinny_fp8_64x32";
  const int splits = choose_splits(a);
  return splits <= 8 ? kSplitNames[splits] : "skinny_fp8_64x128_splitk";
}

}  // namespace

const Variant* variant_skinny_fp8() {
  static const Variant v = {"skinny_fp8_64x32", accepts, launch, name_of, scratch_bytes};
  return &v;
}

}  // namespace tg
