// Registration of the tuned tile kernel (tile_mfma.hpp) for B stored N x K
// (both operands K-contiguous), the layout of the 4096 x 7168 x 16384 BF16
// GEMM reported for the Ascend release in "Getting to know TileLang"
// (six-piece section).  Products with too few tiles to fill the CUs take
// 128 x 128 tiles when K is short, and split K across the workgroups of a
// tile (a one-GPU shard of that product, 4096 x 896 x 16384, has 64 tiles
// of 256 x 224, each split 4 ways).  Grids of one whole wave and a partial
// one may split only the partial wave's tiles.
#include "tile_mfma.hpp"
#include "tile_pp.hpp"

namespace tg {
namespace {

using tile::Mfma16;
using tile::Mfma32;
// wave tile 128 x 112, 16x16x32 MFMAs; B one LDS stage deeper than A
typedef tile::Tile<256, 224, Mfma16, 2, 3> Tile224;
typedef tile::Tile<256, 256, Mfma32> Tile256;  // wave tile 128 x 128, 32x32x16 MFMAs
// wave tile 64 x 64, 16x16x32 MFMAs: three stages of A and of B (96 KiB) for
// grids of at most one workgroup per CU; two of each (64 KiB, two workgroups
// per CU) for larger grids
typedef tile::Tile<128, 128, Mfma16, 3, 3> Tile128;
typedef tile::Tile<128, 128, Mfma16, 2, 2> Tile128x2;
// unsplit 256 x 224 and 256 x 256 tiles run the eight-wave ping-pong form
typedef tile::PPTile<224> PP224;
typedef tile::PPTile<256> PP256;
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

constexpr int64_t kCus = 256;
// Split K on the eight-wave 256 x 224 kernels: at most 7 splits (with 8, the
// combine of the partials spills about 660 VGPRs beside the accumulators).
constexpr int kMaxSplitsPP = 7;
constexpr int64_t kShortK = 128;  // K slices (of 64) up to which small grids take 128 x 128

// A grid of 256 x 224 tiles is small when it fills at most half the CUs.
bool small_grid(const GemmArgs& a) { return 2 * cdiv(a.M, 256) * cdiv(a.N, 224) <= kCus; }

// Split K across a tile's workgroups only for small grids.
//  - 256 x 224 (long K): as many splits as bring the grid to about one
//    workgroup per CU, at most 8, with at least 8 K slices (of 64) per split.
//    Each split past the first adds about two K slices' time to the combine
//    (the last split of a tile reads the others' partials, latency-bound at
//    about 65 GB/s on one CU), so nk / S slices plus 2 (S - 1) is smallest
//    near S = sqrt(nk / 2), the last cap.
//  - 128 x 128 (K of at most kShortK slices): up to one workgroup per CU, at
//    most 8, with at least 16 K slices per split.
// A small grid of either shape is a single wave; the 256 x 256 tile only
// runs grids too large to split.
template <typename Cfg>
int splits_for(const GemmArgs& a) {
  if (std::is_same<Cfg, Tile256>::value || std::is_same<Cfg, Tile128x2>::value) return 1;
  const int64_t tiles = cdiv(a.M, Cfg::BM) * cdiv(a.N, Cfg::BN);
  const int64_t nk = cdiv(a.K, 64);
  int64_t s = kCus / tiles;
  if (s > tile::kMaxSplits) s = tile::kMaxSplits;
  if (!std::is_same<Cfg, Tile128>::value && s > kMaxSplitsPP) s = kMaxSplitsPP;
  if (std::is_same<Cfg, Tile128>::value) {
    if (s > nk / 16) s = nk / 16;
  } else {
    if (2 * tiles > kCus) return 1;
    if (s > nk / 8) s = nk / 8;
    while (s > 1 && 2 * s * s > nk) --s;
  }
  return s < 2 ? 1 : (int)s;
}

// Tile choice.  Small grids (at most half the CUs in 256 x 224 tiles) take
// 128 x 128 tiles when K is at most kShortK slices, or when no scratch is
// at hand to split K: four times the tiles, so fewer or no K splits, and a
// lower fixed cost per tile (measured on 1024^3, 2048^3, 1024 x 1024 x 4096
// and 512 x 512 x 8192: 1.6 to 3.2 times faster than 256 x 224 with split
// K).  Up to 256 of them run with three stages per operand, one workgroup per
// CU (2048^3: 18.3 us against 24.0 with two stages); more run with two
// stages, two workgroups per CU (4096 x 1792 x 4096: 50.4 us against 57.1
// with three).  With longer K the larger tile's lower bytes per FLOP win
// (4096 x 896 x 16384, 2048 x 1024 x 16384) when it may split K.  Other
// grids run in ceil(tiles / 256) waves over the 256 CUs, each wave costing
// about one tile's MFMA work (with 256 x 224 and scratch, a partial second
// wave may have its tiles split over K: tile::tail_splits).  The shape with
// the smaller waves x tile area wins, 256 x 256 on ties (4096 x 7168:
// 256 x 224 gives 512 tiles = 2 full waves, 256 x 256 gives 448 tiles =
// 1.75 waves rounded up to 2).
double cost(const GemmArgs& a, int64_t bm, int64_t bn, bool split_ok) {
  const int64_t tiles = cdiv(a.M, bm) * cdiv(a.N, bn), nk = cdiv(a.K, 64);
  const int s = bn == 224 && split_ok ? tile::tail_splits(tiles, nk, kCus, kMaxSplitsPP) : 1;
  return tile::tail_waves(tiles, nk, kCus, s) * double(bm * bn);
}
enum class Shape { T128, T128x2, T224, T256 };

// A call's plan: tile shape, K splits per tile (splits > 1 with tail: only
// the tiles past the first whole wave are split) and its scratch bytes.
struct Plan {
  Shape shape;
  int splits;
  bool tail;
  size_t bytes;
};

Plan plan_of(const GemmArgs& a, bool split_ok) {
  Plan p{Shape::T256, 1, false, 0};
  if (small_grid(a)) {
    if (split_ok && cdiv(a.K, 64) > kShortK) {
      p.shape = Shape::T224;
      p.splits = splits_for<Tile224>(a);
    } else if (cdiv(a.M, 128) * cdiv(a.N, 128) <= kCus) {
      p.shape = Shape::T128;
      p.splits = split_ok ? splits_for<Tile128>(a) : 1;
    } else {
      p.shape = Shape::T128x2;
    }
  } else if (cost(a, 256, 224, split_ok) < cost(a, 256, 256, split_ok)) {
    p.shape = Shape::T224;
    if (split_ok) {
      p.splits = tile::tail_splits(cdiv(a.M, 256) * cdiv(a.N, 224), cdiv(a.K, 64), kCus,
                                   kMaxSplitsPP);
      p.tail = p.splits > 1;
    }
  }
  if (p.splits > 1) {
    // one counter per split tile in the fixed counter area (at most 4096),
    // then each split's fp32 partial tile
    const int64_t bm = p.shape == Shape::T224 ? 256 : 128, bn = p.shape == Shape::T224 ? 224 : 128;
    const int64_t tiles = cdiv(a.M, bm) * cdiv(a.N, bn);
    const int64_t split_tiles = p.tail ? tiles % kCus : tiles;
    if (split_tiles > kWorkspaceCounters) {
      p.splits = 1;
      p.tail = false;
    } else {
      p.bytes = kWorkspaceCounterBytes + (size_t)(bm * bn * 4) * p.splits * split_tiles;
    }
  }
  return p;
}

// The split plan when `ws` holds its scratch, else the allocation-free one.
Plan choose(const GemmArgs& a, const Scratch& ws) {
  const Plan p = plan_of(a, true);
  if (p.bytes == 0 || scratch_fits(ws, p.bytes)) return p;
  return plan_of(a, false);
}

size_t scratch_bytes(const GemmArgs& a) { return plan_of(a, true).bytes; }

// A split plan of 256 x 224 tiles on the eight-wave kernels, S splits per
// split tile (S is a template parameter of the kernels: one combine per
// kernel).  Tail plans split only the tiles past the first whole wave.
template <int S>
hipError_t launch_pp_split(Op op, const GemmArgs& a, const Plan& p, const Scratch& ws, int tm,
                           int tn, hipStream_t s) {
  int* counters = reinterpret_cast<int*>(ws.ptr);
  float* part = reinterpret_cast<float*>(ws.ptr + kWorkspaceCounterBytes);
  const dim3 block(512);
  if (p.tail) {
    // whole tiles of the first wave, then the split tiles' units
    const int tiles = tm * tn, tail = tiles % (int)kCus, full = tiles - tail;
    const dim3 grid((unsigned)(full + tail * S));
    if (op == Op::BF16)
      hipLaunchKernelGGL((tile::gemm16_pp_tail<__bf16, PP224, S>), grid, block, 0, s, a, tm, tn,
                         full, part, counters);
    else
      hipLaunchKernelGGL((tile::gemm16_pp_tail<_Float16, PP224, S>), grid, block, 0, s, a, tm, tn,
                         full, part, counters);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(tm * tn * S));
  if (op == Op::BF16)
    hipLaunchKernelGGL((tile::gemm16_pp_splitk<__bf16, PP224, S>), grid, block, 0, s, a, tm, tn,
                       part, counters);
  else
    hipLaunchKernelGGL((tile::gemm16_pp_splitk<_Float16, PP224, S>), grid, block, 0, s, a, tm, tn,
                       part, counters);
  return hipGetLastError();
}

template <typename Cfg>
hipError_t launch_cfg(Op op, const GemmArgs& a, const Plan& p, const Scratch& ws, hipStream_t s) {
  const int tm = (int)cdiv(a.M, Cfg::BM), tn = (int)cdiv(a.N, Cfg::BN);
  if constexpr (std::is_same<Cfg, Tile224>::value) {
    if (p.splits > 1) {
      // split-K and partial-wave tiles run the eight-wave form as well; its
      // fp32 partial tile takes the same 256 x 224 x 4 bytes per split
      switch (p.splits) {
        case 2: return launch_pp_split<2>(op, a, p, ws, tm, tn, s);
        case 3: return launch_pp_split<3>(op, a, p, ws, tm, tn, s);
        case 4: return launch_pp_split<4>(op, a, p, ws, tm, tn, s);
        case 5: return launch_pp_split<5>(op, a, p, ws, tm, tn, s);
        case 6: return launch_pp_split<6>(op, a, p, ws, tm, tn, s);
        case 7: return launch_pp_split<7>(op, a, p, ws, tm, tn, s);
        default: return launch_pp_split<kMaxSplitsPP>(op, a, p, ws, tm, tn, s);
      }
    }
  }
  if constexpr (std::is_same<Cfg, Tile128>::value) {
    if (p.splits > 1) {
      int* counters = reinterpret_cast<int*>(ws.ptr);
      float* part = reinterpret_cast<float*>(ws.ptr + kWorkspaceCounterBytes);
      const dim3 grid((unsigned)(tm * tn * p.splits)), block(256);
      if (op == Op::BF16)
        hipLaunchKernelGGL((tile::gemm16_tile_splitk<__bf16, Cfg>), grid, block, 0, s, a, tm, tn,
                           p.splits, part, counters);
      else
        hipLaunchKernelGGL((tile::gemm16_tile_splitk<_Float16, Cfg>), grid, block, 0, s, a, tm,
                           tn, p.splits, part, counters);
      return hipGetLastError();
    }
  }
  const dim3 grid(tm * tn);
  if constexpr (std::is_same<Cfg, Tile224>::value || std::is_same<Cfg, Tile256>::value) {
    // whole-K tiles of the large shapes: eight waves, two per SIMD taking
    // turns at the matrix core (measured in one process on 4096 x 7168 x
    // 16384: 637 us against 693 for the four-wave 256 x 224 kernel; 8192^3:
    // 694 us against 803 for the four-wave 256 x 256 kernel; bit-identical)
    typedef typename std::conditional<std::is_same<Cfg, Tile224>::value, PP224, PP256>::type PP;
    if (op == Op::BF16)
      hipLaunchKernelGGL((tile::gemm16_pp<__bf16, PP>), grid, dim3(512), 0, s, a, tm, tn);
    else
      hipLaunchKernelGGL((tile::gemm16_pp<_Float16, PP>), grid, dim3(512), 0, s, a, tm, tn);
  } else {
    if (op == Op::BF16)
      hipLaunchKernelGGL((tile::gemm16_tile<__bf16, Cfg, false>), grid, dim3(256), 0, s, a, tm,
                         tn);
    else
      hipLaunchKernelGGL((tile::gemm16_tile<_Float16, Cfg, false>), grid, dim3(256), 0, s, a, tm,
                         tn);
  }
  return hipGetLastError();
}

hipError_t launch(Op op, const GemmArgs& a, const Scratch& ws, hipStream_t s) {
  const Plan p = choose(a, ws);
  switch (p.shape) {
    case Shape::T128: return launch_cfg<Tile128>(op, a, p, ws, s);
    case Shape::T128x2: return launch_cfg<Tile128x2>(op, a, p, ws, s);
    case Shape::T224: return launch_cfg<Tile224>(op, a, p, ws, s);
    default: return launch_cfg<Tile256>(op, a, p, ws, s);
  }
}

// plan names by split count (1 .. 8)
const char* const kNames224[] = {"tile_nt_256x224", "tile_nt_256x224", "tile_nt_256x224_splitk2",
                                 "tile_nt_256x224_splitk3", "tile_nt_256x224_splitk4",
                                 "tile_nt_256x224_splitk5", "tile_nt_256x224_splitk6",
                                 "tile_nt_256x224_splitk7", "tile_nt_256x224_splitk8"};
const char* const kNames128[] = {"tile_nt_128x128", "tile_nt_128x128", "tile_nt_128x128_splitk2",
                                 "tile_nt_128x128_splitk3", "tile_nt_128x128_splitk4",
                                 "tile_nt_128x128_splitk5", "tile_nt_128x128_splitk6",
                                 "tile_nt_128x128_splitk7", "tile_nt_128x128_splitk8"};
// ... and by the split count of the tiles of a partial last wave (2 .. 8)
const char* const kTails224[] = {"", "", "tile_nt_256x224_tail2", "tile_nt_256x224_tail3",
                                 "tile_nt_256x224_tail4", "tile_nt_256x224_tail5",
                                 "tile_nt_256x224_tail6", "tile_nt_256x224_tail7",
                                 "tile_nt_256x224_tail8"};
const char* name_of(const GemmArgs& a, const Scratch& ws) {
  const Plan p = choose(a, ws);
  switch (p.shape) {
    case Shape::T128: return kNames128[p.splits];
    case Shape::T128x2: return "tile_nt_128x128_2stage";
    case Shape::T224: return p.tail ? kTails224[p.splits] : kNames224[p.splits];
    default: return "tile_nt_256x256";
  }
}

}  // namespace

const Variant* variant_tile_nt16() {
  static const Variant v = {"tile_nt", accepts, launch, name_of, scratch_bytes};
  return &v;
}

}  // namespace tg
