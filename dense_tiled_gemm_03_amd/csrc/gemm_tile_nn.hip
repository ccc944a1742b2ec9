// Registration of the tuned tile kernel (tile_mfma.hpp) for B stored K x N
// row-major (sbn = 1), the layout of the first-GEMM listing of "Getting to
// know TileLang" and of the 4096^3 BF16 workload.  B tiles are staged as
// [k][n] rows and read with the gfx950 transpose read; 256 x 256 tiles in
// the eight-wave ping-pong form (tile_pp.hpp), 16x16x32 MFMAs (a 4096 x 4096
// C is exactly one wave of 256 tiles).
#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// A K-contiguous and B N-contiguous, 16-byte aligned rows, N a multiple of 8
// (whole 16-byte column chunks); the descriptor ranges (A: one tile of rows,
// B: all K rows of one tile's columns) fit the 31-bit range they use.
bool accepts(Op op, const GemmArgs& a) {
  if (op == Op::FP8) return false;
  if (a.K == 0 || a.K % 8 != 0 || a.N % 8 != 0) return false;
  if (a.sak != 1 || a.sbn != 1) return false;
  if (a.sam % 8 != 0 || a.sbk % 8 != 0) return false;
  if (!aligned16(a.A) || !aligned16(a.B)) return false;
  const int64_t lim = int64_t(1) << 30;
  if (256 * a.sam * 2 + 2 * a.K >= lim || a.K * a.sbk * 2 + 2 * 256 >= lim) return false;
  if (a.M > (int64_t(1) << 24) || a.N > (int64_t(1) << 24)) return false;
  return true;
}

// 256 x 256 tiles in the eight-wave ping-pong form (measured on 4096^3
// with five rotated operand copies: see the design notes).
hipError_t launch(Op op, const GemmArgs& a, const Scratch&, hipStream_t s) {
  typedef tile::PPTile<256> PP;
  const int tm = (int)cdiv(a.M, PP::BM), tn = (int)cdiv(a.N, PP::BN);
  const dim3 grid(tm * tn), block(512);
  if (op == Op::BF16)
    hipLaunchKernelGGL((tile::gemm16_pp<__bf16, PP, true>), grid, block, 0, s, a, tm, tn);
  else
    hipLaunchKernelGGL((tile::gemm16_pp<_Float16, PP, true>), grid, block, 0, s, a, tm, tn);
  return hipGetLastError();
}

}  // namespace

const Variant* variant_tile_nn16() {
  static const Variant v = {"tile_nn_256x256", accepts, launch, nullptr, nullptr};
  return &v;
}

}  // namespace tg
