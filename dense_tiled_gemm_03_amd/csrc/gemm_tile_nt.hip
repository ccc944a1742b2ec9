// Registration of the tuned tile kernel (tile_mfma.hpp) for B stored N x K
// (both operands K-contiguous), the layout of the 4096 x 7168 x 16384 BF16
// GEMM reported for the Ascend release in "Getting to know TileLang"
// (six-piece section).
#include "tile_mfma.hpp"

namespace tg {
namespace {

using tile::Mfma16;
using tile::Mfma32;
typedef tile::Tile<256, 224, Mfma16> Tile224;  // wave tile 128 x 112, 16x16x32 MFMAs
typedef tile::Tile<256, 256, Mfma32> Tile256;  // wave tile 128 x 128, 32x32x16 MFMAs
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
    hipLaunchKernelGGL((tile::gemm16_tile<__bf16, Cfg, false>), grid, block, 0, s, a, tm, tn);
  else
    hipLaunchKernelGGL((tile::gemm16_tile<_Float16, Cfg, false>), grid, block, 0, s, a, tm, tn);
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
