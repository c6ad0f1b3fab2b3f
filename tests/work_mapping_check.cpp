// Host check of the prefill work mapping (prefill_work_item, the device
// header's own code): for every grid it must be a bijection from workgroup
// index to (query tile, pair), so that every output tile is written exactly
// once.  Prints "ok" and exits 0, or names the first failing shape.
#include <cstdio>
#include <vector>

#include "../exact_io_aware_tile_amd/csrc/fa_device.h"

int main() {
  const int qtiles[] = {1, 2, 3, 8, 16, 17, 32};
  const int pairs[] = {1, 7, 8, 12, 16, 24, 40, 64, 128, 512};
  const int groups[] = {1, 2, 3, 4, 8, 16};
  const int chunks[] = {0, 1, 2, 3, 4, 5, 8, 12, 16, 64, 65536};
  long checked = 0;
  for (int nq : qtiles)
    for (int np : pairs)
      for (int g : groups) {
        if (np % g) continue;  // pairs = sequences x heads_q, a multiple of the group
        for (int c : chunks) {
          const int nwg = nq * np;
          std::vector<int> seen(nwg, 0);
          for (int w = 0; w < nwg; ++w) {
            int qt = -1, bh = -1;
            fa::prefill_work_item(nwg, w, nq, g, c, qt, bh);
            if (qt < 0 || qt >= nq || bh < 0 || bh >= np) {
              std::printf("out of range: qtiles %d pairs %d group %d chunk %d w %d -> qt %d bh %d\n", nq, np, g, c,
                          w, qt, bh);
              return 1;
            }
            ++seen[bh * nq + qt];
          }
          for (int i = 0; i < nwg; ++i)
            if (seen[i] != 1) {
              std::printf("not a bijection: qtiles %d pairs %d group %d chunk %d item %d seen %d\n", nq, np, g, c, i,
                          seen[i]);
              return 1;
            }
          ++checked;
        }
      }
  std::printf("ok %ld grids\n", checked);
  return 0;
}
