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
//    registers: 128 x 112 with 16x16x32 MFMAs, 128 x 128 with 32x32x16;
//  - K slice of 64: one LDS row is 128 bytes (eight 16-byte chunks); tiles
//    go HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging);
//    two LDS stages, the next slice's loads in flight while the current one
//    is multiplied;
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

#include "common.hpp"

namespace tg {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int V> using Int = std::integral_constant<int, V>;

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every descriptor's range
constexpr int kXcds = 8;

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

template <int BM_, int BN_, typename MMA_>
struct NtTile {
  typedef MMA_ MMA;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BK = 64;                      // k per LDS stage
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile (2 x 2 waves)
  static constexpr int FM = WTM / MMA::DIM, FN = WTN / MMA::DIM;
  static constexpr int SUBS = BK / MMA::KSTEP;       // MFMA sub-steps per slice
  static constexpr int ROW_BYTES = BK * 2;           // 128
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;  // 1 KiB loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int GM = 4;                       // M-tiles per tile-order group
  static_assert(WTM % MMA::DIM == 0 && WTN % MMA::DIM == 0, "wave tile must fit the MFMA");
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole loads per wave");
  static_assert(FM + FN <= 15, "a sub-step's reads must fit the lgkmcnt counter");
  static_assert(SUBS % 2 == 0, "fragment buffers alternate per sub-step");
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
  typedef typename Cfg::MMA MMA;
  typedef typename MMA::Acc Acc;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUBS = Cfg::SUBS, DIM = MMA::DIM;
  __shared__ __attribute__((aligned(1024))) char lds[2 * Cfg::STAGE_BYTES];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, Cfg::GM, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = w >> 1, wn = w & 1;
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
  // logical chunk (l & 7) ^ swizzle(row) = (l & 7) ^ (4 * (w & 1) + (l >> 4)).
  const int lrow = 8 * w + (lane >> 3);
  const int lchunk = (lane & 7) ^ (4 * (w & 1) + (lane >> 4));
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

  // Reads: fragment row r = (DIM-aligned base) + (l % DIM), chunk
  // s * (KSTEP / 8) + l / DIM of the 64-wide slice for sub-step s, at chunk
  // position chunk ^ swizzle(r) = chunk ^ ((l >> 1) & 7).
  const int sw = (lane >> 1) & 7;
  const int rd_lane = (lane % DIM) * Cfg::ROW_BYTES;
  const int rd_chunk = lane / DIM;
  const int a_rd = wm * Cfg::WTM * Cfg::ROW_BYTES + rd_lane;
  const int b_rd = Cfg::A_BYTES + wn * Cfg::WTN * Cfg::ROW_BYTES + rd_lane;

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < MMA::NACC; ++v) acc[i][j][v] = 0.0f;

  // Fragments of one sub-step, double-buffered.
  T8 fa[2][FM], fb[2][FN];
  constexpr int NRD = FM + FN;                       // LDS reads per sub-step
  constexpr int NLD = Cfg::A_LOADS + Cfg::B_LOADS;   // LDS-direct loads per slice
  static_assert(NRD <= FM * FN && NLD <= FM * FN, "one read and one load per MFMA");
  // The r-th read of a sub-step, in the order the MFMAs consume fragments:
  // a0, b0 .. b[FN-1], a1 .. a[FM-1].
  auto read_one = [&](int buf, const char* base, int r) {
    if (r == 0)
      fa[buf][0] = *reinterpret_cast<const T8*>(base + a_rd);
    else if (r <= FN)
      fb[buf][r - 1] = *reinterpret_cast<const T8*>(base + b_rd + (r - 1) * DIM * Cfg::ROW_BYTES);
    else
      fa[buf][r - FN] = *reinterpret_cast<const T8*>(base + a_rd + (r - FN) * DIM * Cfg::ROW_BYTES);
  };
  auto frag_base = [&](int st, int sub) {
    return lds + st * Cfg::STAGE_BYTES + ((sub * (MMA::KSTEP / 8) + rd_chunk) ^ sw) * 16;
  };
  // keeps the scheduler from moving work across it (one wave per SIMD issues
  // everything in order, so the source order below is the issue order)
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // One sub-step: the MFMAs on fragment buffer `cur`; after the n-th MFMA,
  // the n-th read of the next sub-step (into buffer cur ^ 1, from `next`)
  // and, when LOADS, the LDS-direct loads of the slice at ld_k0 into stage
  // ld_st, spread over the sub-step.  Spreading reads and loads over the MFMA stream hides their
  // issue cycles under MFMA execution and keeps at most one sub-step of
  // reads (<= 15, the lgkmcnt limit) in flight.
  auto substep = [&](auto loads_c, int cur, const char* next, int ld_st, int ld_k0) {
    constexpr bool LOADS = decltype(loads_c)::value;
    const bool kin = ld_k0 + 8 * lchunk < K;
    char* ld_base = lds + ld_st * Cfg::STAGE_BYTES;
#pragma unroll
    for (int n = 0; n < FM * FN; ++n) {
      const int i = n / FN, j = n % FN;
      acc[i][j] = MMA::mma(fa[cur][i], fb[cur][j], acc[i][j]);
      if (n < NRD) read_one(cur ^ 1, next, n);
      if constexpr (LOADS) {
        // load q goes after MFMA q * FM * FN / NLD: spread evenly, since a CU
        // moves 64 B per clock from L2 and a burst of loads would stall the
        // wave's issue (and with it the MFMAs) behind a full memory queue
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
          if (q * FM * FN / NLD != n) continue;
          if (q < Cfg::A_LOADS)
            load_lds16(ra, ld_base + (4 * q + w) * 1024,
                       kin ? a_lane + q * a_step + 2 * ld_k0 : kOutOfRange);
          else
            load_lds16(rb, ld_base + Cfg::A_BYTES + (4 * (q - Cfg::A_LOADS) + w) * 1024,
                       kin ? b_lane + (q - Cfg::A_LOADS) * b_step + 2 * ld_k0 : kOutOfRange);
        }
      }
      fence();
    }
  };

  // Pipeline, per slice kt in stage st = kt & 1 (sub-steps s = 0 .. SUBS-1):
  //   s < SUBS-1: MFMAs of sub-step s | reads of sub-step s+1;
  //   then: wait for this wave's loads of slice kt+1 and barrier (after it,
  //     slice kt+1 is in LDS for every wave, and every wave's reads of stage
  //     st have returned -- the last sub-step needs them now anyway);
  //   s = SUBS-1: MFMAs | reads of sub-step 0 of kt+1 | loads of slice
  //     kt+2 -> stage st.
  // Slices at or past K are fetched with out-of-range offsets: they move no
  // data, fill the idle stage with zeros and keep the loop free of branches.
  const int nk = (K + BK - 1) / BK;
  load_stage(0, 0);
  load_stage(1, BK);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
  __syncthreads();
  {
    const char* b0 = frag_base(0, 0);
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(0, b0, r);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
#pragma unroll
    for (int sub = 0; sub < SUBS - 1; ++sub) {
      fence();
      substep(std::false_type(), sub & 1, frag_base(st, sub + 1), 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    fence();
    substep(std::true_type(), (SUBS - 1) & 1, frag_base(st ^ 1, 0), st, (kt + 2) * BK);
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

typedef NtTile<256, 224, Mfma16> Tile224;  // wave tile 128 x 112, 16x16x32 MFMAs
typedef NtTile<256, 256, Mfma32> Tile256;  // wave tile 128 x 128, 32x32x16 MFMAs

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
