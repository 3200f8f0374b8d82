// The workgroup -> (head, tile rank) map of the kernels' 1-D grids, checked
// on the host over many shapes (see tests/test_grid_tile.py): for every
// number of heads, tiles per head, dispatch-group size and tail-group size,
// the map must be a bijection from the grid onto heads x ranks (every tile
// computed exactly once), with XCD grouping keep every head on one XCD
// (workgroup b runs on XCD b mod 8), and inside each dispatch group hand out
// ranks in ascending order (rank 0 is a causal head's longest tile).
// Exit status 0 = every case held.
#include <cstdio>
#include <vector>

#include "fa_device.h"

int main() {
  long cases = 0, failures = 0;
  const int ntiles_list[] = {1, 2, 3, 4, 7, 8, 32, 64, 65, 256};
  const int groups[] = {1, 2, 4, 8, 16};
  for (int heads = 1; heads <= 72; ++heads)
    for (int xcd = 0; xcd < 2; ++xcd) {
      if (xcd && heads % 8) continue;
      for (int nt : ntiles_list)
        for (int group : groups)
          for (int tail : {0, 1, 2, 3, 5, heads / (xcd ? 8 : 1), heads + 3}) {
            ++cases;
            const int n = heads * nt;
            std::vector<int> seen((size_t)n, 0);
            // last rank handed out so far per (lane, group id), for the ordering check
            bool ok = true;
            for (int b = 0; b < n && ok; ++b) {
              int bh = -1, r = -1;
              fa::grid_tile(b, heads, nt, xcd != 0, group, tail, bh, r);
              if (bh < 0 || bh >= heads || r < 0 || r >= nt) { ok = false; break; }
              if (xcd && bh % 8 != b % 8) { ok = false; break; }
              if (seen[(size_t)bh * nt + r]++) { ok = false; break; }
            }
            // ascending ranks: along one XCD's sequence, a head's ranks never go down
            if (ok) {
              const int lanes = xcd ? 8 : 1;
              for (int x = 0; x < lanes && ok; ++x) {
                std::vector<int> last((size_t)heads, -1);
                for (int b = x; b < n && ok; b += lanes) {
                  int bh, r;
                  fa::grid_tile(b, heads, nt, xcd != 0, group, tail, bh, r);
                  if (r < last[(size_t)bh]) ok = false;
                  last[(size_t)bh] = r;
                }
              }
            }
            if (!ok) {
              if (++failures <= 10)
                std::fprintf(stderr, "FAIL heads=%d ntiles=%d xcd=%d group=%d tail=%d\n", heads, nt, xcd,
                             group, tail);
            }
          }
    }
  if (failures) {
    std::fprintf(stderr, "%ld of %ld cases failed\n", failures, cases);
    return 1;
  }
  std::printf("grid_tile: %ld cases hold\n", cases);
  return 0;
}
