// Host-side check of tile::tail_unit, the workgroup map of grids with whole
// tiles and split units: over many grid sizes, every whole tile and every
// split unit is taken by exactly one workgroup, and on each XCD (workgroup
// b runs on XCD b % 8) the whole tiles come before the split units.
// Prints "ok <grids>" or the first failure, and exits non-zero on failure.
#include "../dense_tiled_gemm_03_amd/csrc/tile_mfma.hpp"

#include <cstdio>
#include <vector>

int main() {
  long grids = 0;
  for (int full = 0; full <= 3000; full += (full < 600 ? 1 : 37))
    for (int units = 1; units <= 2048; units += (units < 300 ? 1 : 41)) {
      const int G = full + units;
      std::vector<int> seen_whole(full, 0), seen_unit(units, 0);
      std::vector<bool> split_started(8, false);
      for (int b = 0; b < G; ++b) {
        int id = -1;
        const bool whole = tg::tile::tail_unit(b, G, full, id);
        const int x = b % 8;
        if (whole) {
          if (id < 0 || id >= full || seen_whole[id]++ || split_started[x]) {
            printf("fail: full=%d units=%d b=%d whole id=%d\n", full, units, b, id);
            return 1;
          }
        } else {
          if (id < 0 || id >= units || seen_unit[id]++) {
            printf("fail: full=%d units=%d b=%d unit id=%d\n", full, units, b, id);
            return 1;
          }
          split_started[x] = true;
        }
      }
      ++grids;
    }
  printf("ok %ld\n", grids);
  return 0;
}
