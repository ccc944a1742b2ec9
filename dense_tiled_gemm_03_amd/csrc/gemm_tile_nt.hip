// Tuned kernel for fp16 / bf16 C = A * B when both operands are K-contiguous:
// A row-major (M x K, sak = 1) and B stored N x K (sbk = 1), the layout of the
// 4096 x 7168 x 16384 BF16 GEMM reported for the Ascend release in "Getting to
// know TileLang" (six-piece section).
//
// The structure is the tile loop of "TileKernels deep dive" section 3.1 and
// the first-GEMM listing of "Getting to know TileLang" (one output tile per
// workgroup, operand tiles staged in on-chip memory per K slice with a
// multi-stage pipeline, an fp32 accumulator copied to C once with a cast),
// laid out for gfx950:
//  - workgroup tile BM x BN (256 x 224 or 256 x 256), 4 waves in a 2 x 2
//    grid, each wave owning a (BM/2) x (BN/2) block of fp32 accumulators in
//    registers, updated with 16x16x32 MFMAs;
//  - K slice of 64: one LDS row is 128 bytes (eight 16-byte chunks); tiles
//    go HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging);
//    two LDS stages, the next slice's loads in flight while the current one
//    is multiplied;
//  - LDS chunk swizzle: chunk c of row r sits at chunk position
//    c ^ ((r & 7) ^ ((r >> 3) & 1)), so the 16 rows one 16-lane group reads
//    with ds_read_b128 fall on distinct bank groups;
//  - edges: the buffer descriptor of each operand tile ends at the last valid
//    element, so rows past M (or N) read as zero; chunks past K get an
//    out-of-range offset and read as zero; the epilogue masks the stores;
//  - tile order: workgroups the hardware places on one XCD (blockIdx % 8)
//    get consecutive tile ids, walked in groups of GM M-tiles so concurrent
//    tiles on one XCD share A rows and B columns in that XCD's L2.
#include "common.hpp"

namespace tg {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every descriptor's range
constexpr int kXcds = 8;

template <int BM_, int BN_, int WAVES_M_>
struct NtTile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BK = 64;                   // k per LDS stage
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = 4 / WAVES_M_;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;            // 32 x 32 fragments
  static constexpr int ROW_BYTES = BK * 2;         // 128
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;  // 1 KiB loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int GM = 4;                     // M-tiles per tile-order group
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole loads per wave");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, const void* lds,
                                           uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// Tile id -> (tile row, tile column): XCD-contiguous ids, then groups of GM
// tile rows walked row-fastest.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int gm_size, int& tm,
                                            int& tn) {
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcds, local = b / kXcds;
  const int per = G / kXcds, rem = G % kXcds;
  const int id = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int span = gm_size * tiles_n;
  const int group = id / span, first_m = group * gm_size;
  const int gm = min(gm_size, tiles_m - first_m);
  const int in = id - group * span;
  tm = first_m + in % gm;
  tn = in / gm;
}

template <typename T, typename Cfg>
__global__ __launch_bounds__(256) void gemm16_nt(GemmArgs a, int tiles_m, int tiles_n) {
  typedef typename Elem<T>::x8 T8;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  __shared__ __attribute__((aligned(1024))) char lds[2 * Cfg::STAGE_BYTES];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
  const int K = (int)a.K;
  const uint32_t lda = (uint32_t)a.sam, ldb = (uint32_t)a.sbn;

  // Operand tiles as buffer descriptors that end at the last valid element.
  const int rows_a = (int)min<int64_t>(BM, a.M - m0), rows_b = (int)min<int64_t>(BN, a.N - n0);
  const T* Ab = static_cast<const T*>(a.A) + m0 * a.sam;
  const T* Bb = static_cast<const T*>(a.B) + n0 * a.sbn;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, (uint32_t)(((rows_a - 1) * lda + K) * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, (uint32_t)(((rows_b - 1) * ldb + K) * 2));

  // Loads: wave w's i-th load fills LDS rows 8*(4i + w) .. +7 of a tile; lane
  // l writes row 8*(4i + w) + (l >> 3), chunk position l & 7, so it fetches
  // logical chunk (l & 7) ^ swizzle(row) = (l & 7) ^ (l >> 3) ^ (w & 1).
  const int lrow = 8 * w + (lane >> 3);
  const int lchunk = (lane & 7) ^ (lane >> 3) ^ (w & 1);
  const uint32_t a_lane = (uint32_t)lrow * lda * 2 + 16 * lchunk;
  const uint32_t b_lane = (uint32_t)lrow * ldb * 2 + 16 * lchunk;
  const uint32_t a_step = 32 * lda * 2, b_step = 32 * ldb * 2;  // 32 rows per load index

  auto load_stage = [&](int st, int k0) {
    const bool kin = k0 + 8 * lchunk < K;
    char* base = lds + st * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
      load_lds16(ra, base + (4 * i + w) * 1024, kin ? a_lane + i * a_step + 2 * k0 : kOutOfRange);
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i)
      load_lds16(rb, base + Cfg::A_BYTES + (4 * i + w) * 1024,
                 kin ? b_lane + i * b_step + 2 * k0 : kOutOfRange);
  };

  // Reads: a 32 x 16 fragment row r = (32-aligned base) + (l & 31), chunk
  // 2s + (l >> 5) of the 64-wide slice for k16 sub-step s, at chunk position
  // chunk ^ swizzle(r) = chunk ^ swizzle(l & 15).
  const int sw = (lane & 7) ^ ((lane >> 3) & 1);
  int rd[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
    rd[s4] = (lane & 31) * Cfg::ROW_BYTES + ((2 * s4 + (lane >> 5)) ^ sw) * 16;
  const int a_rd = wm * Cfg::WTM * Cfg::ROW_BYTES;
  const int b_rd = Cfg::A_BYTES + wn * Cfg::WTN * Cfg::ROW_BYTES;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragments of one k16 sub-step, double-buffered.
  T8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](int buf, int st, int sub) {
    const char* base = lds + st * Cfg::STAGE_BYTES + rd[sub];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[buf][i] = *reinterpret_cast<const T8*>(base + a_rd + i * 32 * Cfg::ROW_BYTES);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[buf][j] = *reinterpret_cast<const T8*>(base + b_rd + j * 32 * Cfg::ROW_BYTES);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[buf][i], fb[buf][j], acc[i][j]);
  };

  // Pipeline, per 64-wide slice kt in stage st = kt & 1:
  //   loads of slice kt+1 -> stage st^1 (that stage was last read in slice
  //   kt-1, before the previous barrier);
  //   each k16 sub-step's fragments are read while the previous sub-step's
  //   MFMAs run; before sub-step 0 of slice kt+1 is read, wait for slice
  //   kt+1's loads and pass the barrier.
  // The last slice's prefetch asks for k >= K: every chunk is out of range,
  // so it moves no data, fills the idle stage with zeros and keeps the loop
  // body free of branches.
  // keeps the scheduler from moving a sub-step's reads behind the MFMAs
  // that are meant to hide them
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  const int nk = (K + BK - 1) / BK;
  load_stage(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    load_stage(st ^ 1, (kt + 1) * BK);
    read_frags(1, st, 1);
    fence();
    mfmas(0);
    fence();
    read_frags(0, st, 2);
    fence();
    mfmas(1);
    fence();
    read_frags(1, st, 3);
    fence();
    mfmas(0);
    fence();
    // this wave's LDS-direct loads of slice kt+1 have landed (and its reads
    // of slice kt have returned); after the barrier every wave's have
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    read_frags(0, st ^ 1, 0);
    fence();
    mfmas(1);
    fence();
  }

  // Epilogue: lane l holds column (l & 31), rows 8 * (v / 4) + 4 * (l >> 5)
  // + (v % 4) of each 32 x 32 fragment; round to the output type and store
  // inside M x N.
  T* C = static_cast<T*>(a.C);
  const int64_t row0 = m0 + wm * Cfg::WTM + 4 * (lane >> 5);
  const int64_t col0 = n0 + wn * Cfg::WTN + (lane & 31);
  if (m0 + BM <= a.M && n0 + BN <= a.N) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          C[(row0 + i * 32 + 8 * (v >> 2) + (v & 3)) * a.scm + col0 + j * 32] =
              to_out<T>(acc[i][j][v]);
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = row0 + i * 32 + 8 * (v >> 2) + (v & 3), col = col0 + j * 32;
          if (row < a.M && col < a.N) C[row * a.scm + col] = to_out<T>(acc[i][j][v]);
        }
  }
}

typedef NtTile<256, 224, 4> Tile224;  // waves 4 x 1, wave tile 64 x 224
typedef NtTile<256, 256, 2> Tile256;  // waves 2 x 2, wave tile 128 x 128

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Both operands K-contiguous with 16-byte aligned rows; offsets inside one
// operand tile fit the 31-bit range the descriptors use.
bool accepts(Op op, const GemmArgs& a) {
  if (op == Op::FP8) return false;
  if (a.K == 0 || a.K % 8 != 0) return false;
  if (a.sak != 1 || a.sbk != 1) return false;
  if (a.sam % 8 != 0 || a.sbn % 8 != 0) return false;
  if (!aligned16(a.A) || !aligned16(a.B)) return false;
  const int64_t lim = int64_t(1) << 30;
  if (256 * a.sam * 2 + 2 * a.K >= lim || 256 * a.sbn * 2 + 2 * a.K >= lim) return false;
  if (a.M > (int64_t(1) << 24) || a.N > (int64_t(1) << 24)) return false;
  return true;
}

template <typename Cfg>
hipError_t launch_cfg(Op op, const GemmArgs& a, hipStream_t s) {
  const int tm = (int)cdiv(a.M, Cfg::BM), tn = (int)cdiv(a.N, Cfg::BN);
  const dim3 grid(tm * tn), block(256);
  if (op == Op::BF16)
    hipLaunchKernelGGL((gemm16_nt<__bf16, Cfg>), grid, block, 0, s, a, tm, tn);
  else
    hipLaunchKernelGGL((gemm16_nt<_Float16, Cfg>), grid, block, 0, s, a, tm, tn);
  return hipGetLastError();
}

// Tile choice: the grid runs in ceil(tiles / 256) waves over the 256 CUs and
// each wave costs about one tile's MFMA work, so pick the shape with the
// smaller waves x tile area (4096 x 7168: 256 x 224 gives 512 tiles = 2 full
// waves, 256 x 256 gives 448 tiles = 1.75 waves rounded up to 2).
constexpr int64_t kCus = 256;
int64_t cost(const GemmArgs& a, int64_t bm, int64_t bn) {
  return cdiv(cdiv(a.M, bm) * cdiv(a.N, bn), kCus) * bm * bn;
}
bool use224(const GemmArgs& a) { return cost(a, 256, 224) < cost(a, 256, 256); }

hipError_t launch(Op op, const GemmArgs& a, hipStream_t s) {
  return use224(a) ? launch_cfg<Tile224>(op, a, s) : launch_cfg<Tile256>(op, a, s);
}

const char* name_of(const GemmArgs& a) { return use224(a) ? "tile_nt_256x224" : "tile_nt_256x256"; }

}  // namespace

const Variant* variant_tile_nt16() {
  static const Variant v = {"tile_nt", accepts, launch, name_of};
  return &v;
}

}  // namespace tg
