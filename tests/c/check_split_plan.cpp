// Host check of the persistent GEMM's split schedule (split_plan and
// split_range in fine_grained_fp8_amd/csrc/kernels.hpp): prints the plan for
// a grid of launches, one line each, for the Python test to compare with its
// own statement of the rule, and counts violations of the invariants every
// plan must meet:
//  * whole tiles + split tiles = tiles; split_tiles * split <= min(grid, slots)
//  * a split happens only when tiles > grid and the leftover fills at most
//    half of a round
//  * the pieces of a tile cover K blocks [0, kb) exactly, in order, each
//    non-empty, every boundary but the last on a multiple of 4
// Built with g++ against the HIP headers; no device code.
#include <cstdio>

#include "kernels.hpp"

int main() {
  const long tiles_list[] = {1, 7, 8, 255, 256, 257, 300, 383, 384, 385, 511, 512, 896, 1048, 2304, 4032, 5000};
  const long grid_list[] = {8, 64, 248, 256, 304};
  const int kb_list[] = {1, 2, 3, 4, 5, 7, 8, 9, 14, 32, 56, 144, 1000};
  const long slots_list[] = {0, 64, 256, 1024};
  long lines = 0, violations = 0;
  for (long tiles : tiles_list)
    for (long grid : grid_list)
      for (int kb : kb_list)
        for (long slots : slots_list) {
          const fp8bs::SplitPlan s = fp8bs::split_plan(tiles, grid, kb, slots);
          printf("%ld %ld %d %ld %ld %ld %d %d\n", tiles, grid, kb, slots, (long)s.dp_tiles, (long)s.split_tiles,
                 s.split, s.rounds);
          ++lines;
          if (s.dp_tiles + s.split_tiles != tiles) ++violations;
          if (s.split_tiles * s.split > (grid < slots ? grid : slots) && s.split > 1) ++violations;
          if (s.split > 1) {
            if (tiles <= grid || 2 * (tiles % grid) > grid || s.split_tiles != tiles % grid) ++violations;
            int prev = 0;
            for (int piece = 0; piece < s.split; ++piece) {
              int lo, hi;
              fp8bs::split_range(s, piece, kb, lo, hi);
              if (lo != prev || hi <= lo) ++violations;
              if (piece + 1 < s.split && hi % 4 != 0) ++violations;
              prev = hi;
            }
            if (prev != kb) ++violations;
          } else if (s.split_tiles != 0 || s.dp_tiles != tiles) {
            ++violations;
          }
        }
  printf("lines=%ld violations=%ld\n", lines, violations);
  return violations == 0 ? 0 : 1;
}
