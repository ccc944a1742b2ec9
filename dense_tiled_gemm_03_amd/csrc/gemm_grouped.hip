// Grouped fp16 / bf16 product: G independent products that share N and K,
// each with its own number of rows -- the grouped GEMM among the TileLang
// examples ("Getting to know TileLang", operator-coverage section; used for
// the experts of a mixture-of-experts layer, "TileKernels deep dive"
// section 5).  For g < G:
//   C[rows r0_g .. r0_{g+1}) = A[rows r0_g .. r0_{g+1}) * B_g
// with A row-major (K-contiguous), B_g = B + g * sbg stored N x K
// (K-contiguous, leading dimension ldb), C row-major.
//
// One launch covers every group: the tiles of all groups are numbered
// group by group (a group of M_g rows has ceil(M_g / BM) * ceil(N / BN)
// tiles), each workgroup finds its group in a table of first tile ids passed
// with the kernel arguments, re-bases A, B_g and C on the group and runs the
// N x K tile kernel's K loop and epilogue (its eight-wave form) on its tile.  Calls the tile
// kernel does not take (strides, alignment, more than kMaxGroups groups) run
// group by group through tg_gemm_f16 / tg_gemm_bf16.
#include "../../include/tg_gemm.h"

#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

// One group tile per workgroup, in the eight-wave ping-pong form of the
// N x K tile kernel (tile_pp.hpp).
template <typename T, typename Cfg>
__global__ __launch_bounds__(512) void gemm16_grouped(GemmArgs a, GroupTable gt) {
  int g, tm, tn;
  tile::group_coords(gt, Cfg::BM, Cfg::GM, g, tm, tn);
  const int64_t rows = gt.row0[g + 1] - gt.row0[g];
  GemmArgs ag = a;
  ag.M = rows;
  ag.A = static_cast<const T*>(a.A) + gt.row0[g] * a.sam;
  ag.B = static_cast<const T*>(a.B) + g * gt.sbg;
  ag.C = static_cast<T*>(a.C) + gt.row0[g] * a.scm;
  tile::pp_body<T, Cfg>(ag, tm, tn);
}

typedef tile::PPTile<224> Tile224;
typedef tile::PPTile<256> Tile256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct Call {
  int64_t G;
  const int64_t* off;
  int64_t N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb, sbg;
  void* C;
  int64_t ldc;
};

tg_status validate(const Call& c) {
  if (c.G < 0 || c.N < 0 || c.K < 0 || c.lda < 0 || c.ldb < 0 || c.sbg < 0 || c.ldc < 0)
    return TG_ERR_INVALID_VALUE;
  if (c.G == 0) return TG_SUCCESS;
  if (c.off == nullptr) return TG_ERR_INVALID_VALUE;
  if (c.off[0] < 0) return TG_ERR_INVALID_VALUE;
  for (int64_t g = 0; g < c.G; ++g)
    if (c.off[g + 1] < c.off[g]) return TG_ERR_INVALID_VALUE;
  const int64_t rows = c.off[c.G];
  if (rows == 0 || c.N == 0) return TG_SUCCESS;
  if (c.C == nullptr) return TG_ERR_INVALID_VALUE;
  if (c.K > 0 && (c.A == nullptr || c.B == nullptr)) return TG_ERR_INVALID_VALUE;
  if ((rows > 1 && (c.lda < c.K || c.ldc < c.N)) || (c.N > 1 && c.ldb < c.K))
    return TG_ERR_INVALID_VALUE;
  int64_t r;
  if (__builtin_mul_overflow(rows - 1, c.lda, &r) || __builtin_mul_overflow(rows - 1, c.ldc, &r) ||
      __builtin_mul_overflow(c.N - 1, c.ldb, &r) || __builtin_mul_overflow(c.G - 1, c.sbg, &r))
    return TG_ERR_INVALID_VALUE;
  // element extents of A, B and C; byte addresses must not overflow either
  const int64_t lim = int64_t(1) << 61;
  int64_t ea, eb, ec;
  if (__builtin_add_overflow((rows - 1) * c.lda, c.K, &ea) ||
      __builtin_add_overflow((c.G - 1) * c.sbg, (c.N - 1) * c.ldb + c.K, &eb) ||
      __builtin_add_overflow((rows - 1) * c.ldc, c.N, &ec) || ea >= lim || eb >= lim || ec >= lim ||
      c.off[c.G] >= lim)
    return TG_ERR_INVALID_VALUE;
  return TG_SUCCESS;
}

// The tiled launch takes: at most kMaxGroups groups, K a multiple of 8,
// 16-byte aligned rows and group bases, offsets inside a tile within the
// descriptors' range, fewer than 2^31 tiles.
bool tiled(const Call& c) {
  if (c.G > kMaxGroups || c.K == 0 || c.K % 8 != 0) return false;
  if (c.lda % 8 != 0 || c.ldb % 8 != 0 || c.sbg % 8 != 0) return false;
  if (!aligned16(c.A) || !aligned16(c.B)) return false;
  const int64_t lim = int64_t(1) << 30;
  if (256 * c.lda * 2 + 2 * c.K >= lim || 256 * c.ldb * 2 + 2 * c.K >= lim) return false;
  if (c.N > (int64_t(1) << 24)) return false;
  for (int64_t g = 0; g < c.G; ++g)
    if (c.off[g + 1] - c.off[g] > (int64_t(1) << 24)) return false;
  return true;
}

// Tile shape by the same wave-count cost as the single product, over all
// groups' tiles.
int64_t total_tiles(const Call& c, int bm, int bn) {
  int64_t t = 0;
  for (int64_t g = 0; g < c.G; ++g) t += cdiv(c.off[g + 1] - c.off[g], bm) * cdiv(c.N, bn);
  return t;
}
bool use224(const Call& c) {
  const int64_t cus = 256;
  return cdiv(total_tiles(c, 256, 224), cus) * 224 < cdiv(total_tiles(c, 256, 256), cus) * 256;
}

template <typename T, typename Cfg>
tg_status launch_grouped(const Call& c, hipStream_t s) {
  GroupTable gt;
  gt.G = (int)c.G;
  gt.tiles_n = (int)cdiv(c.N, Cfg::BN);
  gt.sbg = c.sbg;
  gt.ssbg = 0;
  int64_t tiles = 0;
  for (int64_t g = 0; g <= c.G; ++g) {
    gt.row0[g] = c.off[g] - c.off[0];
    gt.tile0[g] = (int)tiles;
    if (g < c.G) tiles += cdiv(c.off[g + 1] - c.off[g], Cfg::BM) * gt.tiles_n;
  }
  if (tiles >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
  const GemmArgs a{c.off[c.G] - c.off[0], c.N, c.K,
                   static_cast<const T*>(c.A) + c.off[0] * c.lda, c.lda, 1, c.B, 1, c.ldb,
                   nullptr, 0, 0, nullptr, 0, 0,
                   static_cast<T*>(c.C) + c.off[0] * c.ldc, c.ldc};
  hipLaunchKernelGGL((gemm16_grouped<T, Cfg>), dim3((unsigned)tiles), dim3(512), 0, s, a, gt);
  return hipGetLastError() == hipSuccess ? TG_SUCCESS : TG_ERR_LAUNCH;
}

template <typename T>
tg_status run(const Call& c, tg_stream_t stream) {
  tg_status st = validate(c);
  if (st != TG_SUCCESS || c.G == 0 || c.off[c.G] == c.off[0] || c.N == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tiled(c))
    return use224(c) ? launch_grouped<T, Tile224>(c, s) : launch_grouped<T, Tile256>(c, s);
  // group by group through the general entry point
  for (int64_t g = 0; g < c.G; ++g) {
    const int64_t m = c.off[g + 1] - c.off[g];
    if (m == 0) continue;
    const T* Ag = static_cast<const T*>(c.A) + c.off[g] * c.lda;
    const T* Bg = static_cast<const T*>(c.B) + g * c.sbg;
    T* Cg = static_cast<T*>(c.C) + c.off[g] * c.ldc;
    st = std::is_same<T, __bf16>::value
             ? tg_gemm_bf16(m, c.N, c.K, Ag, c.lda, 1, Bg, 1, c.ldb, Cg, c.ldc, 1, stream)
             : tg_gemm_f16(m, c.N, c.K, Ag, c.lda, 1, Bg, 1, c.ldb, Cg, c.ldc, 1, stream);
    if (st != TG_SUCCESS) return st;
  }
  return TG_SUCCESS;
}

const char* plan(const Call& c) {
  if (validate(c) != TG_SUCCESS) return nullptr;
  if (c.G == 0 || c.off[c.G] == c.off[0] || c.N == 0) return "none";
  if (!tiled(c)) return "per_group";
  return use224(c) ? "grouped_tile_nt_256x224" : "grouped_tile_nt_256x256";
}

}  // namespace
}  // namespace tg

extern "C" {

tg_status tg_gemm_grouped_f16(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb, int64_t sbg,
                              void* C, int64_t ldc, tg_stream_t stream) {
  return tg::run<_Float16>(tg::Call{G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc}, stream);
}

tg_status tg_gemm_grouped_bf16(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                               const void* A, int64_t lda, const void* B, int64_t ldb, int64_t sbg,
                               void* C, int64_t ldc, tg_stream_t stream) {
  return tg::run<__bf16>(tg::Call{G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc}, stream);
}

const char* tg_gemm_grouped_plan(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                                 const void* A, int64_t lda, const void* B, int64_t ldb,
                                 int64_t sbg, void* C, int64_t ldc) {
  return tg::plan(tg::Call{G, offsets, N, K, A, lda, B, ldb, sbg, C, ldc});
}

}  // extern "C"
