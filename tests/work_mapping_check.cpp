// Host check of the prefill work mapping (fa_workmap.h, the code the kernels
// run).  For every grid it must be a bijection from workgroup index to
// (query tile, pair), so that every output tile is written exactly once, and
// it must equal the same order written with plain integer divisions.  The
// multiply-and-shift division it uses is checked against '/' exhaustively
// for small operands and on edge and random operands up to 2^31 - 1.  Prints
// "ok" and exits 0, or names the first failure.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "../exact_io_aware_tile_amd/csrc/fa_workmap.h"

// The order with plain divisions: XCD x = w % 8 takes pairs of GQA groups
// g = x (mod 8), its workgroup of rank j = w / 8 runs query tile
// num_qtiles - 1 - (its round), heaviest first, `chunk` pairs at a time.
static void plain_order(int nwg, int w, int num_qtiles, int group, int chunk, int& qt, int& bh) {
  const int npairs = nwg / num_qtiles;
  if ((npairs / group) % 8 == 0 && npairs % group == 0) {
    const int px = npairs / 8;
    const int j = w / 8;
    int k;
    if (chunk > 0) {
      const int c0 = j / (chunk * num_qtiles) * chunk;
      const int cn = chunk < px - c0 ? chunk : px - c0;
      const int r = j - c0 * num_qtiles;
      k = c0 + r % cn;
      qt = num_qtiles - 1 - r / cn;
    } else {
      k = j % px;
      qt = num_qtiles - 1 - j / px;
    }
    bh = ((k / group) * 8 + w % 8) * group + k % group;
  } else {
    qt = num_qtiles - 1 - (w % num_qtiles);
    bh = w / num_qtiles;
  }
}

static bool check_div(int32_t n, int32_t d) {
  const int32_t q = fa::idiv(n, fa::make_intdiv(d));
  if (q != n / d) {
    std::printf("idiv wrong: %d / %d -> %d, expected %d\n", n, d, q, n / d);
    return false;
  }
  return true;
}

int main() {
  // Division: every n < 2^14 by every d < 2^10, then edges and random pairs.
  for (int32_t d = 1; d < 1024; ++d)
    for (int32_t n = 0; n < 16384; ++n)
      if (!check_div(n, d)) return 1;
  std::mt19937_64 rng(12345);
  const int32_t big = 0x7fffffff;
  for (int i = 0; i < 2000000; ++i) {
    const int32_t d = 1 + (int32_t)(rng() % (uint64_t)big);
    const int32_t n = (int32_t)(rng() % ((uint64_t)big + 1));
    if (!check_div(n, d) || !check_div(big, d) || !check_div(big - (big % d), d) || !check_div(d - 1, d) ||
        !check_div(d, d))
      return 1;
  }
  for (int32_t l = 0; l < 31; ++l) {  // powers of two and their neighbours
    const int32_t p = (int32_t)(int64_t(1) << l);
    for (int32_t d : {p, p + 1, p - 1 > 0 ? p - 1 : 1})
      if (!check_div(big, d) || !check_div(big - 1, d) || !check_div(0, d)) return 1;
  }

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
          const fa::WorkMap m = fa::make_workmap(nwg, nq, g, c);
          std::vector<int> seen(nwg, 0);
          for (int w = 0; w < nwg; ++w) {
            int qt = -1, bh = -1, qt0 = -1, bh0 = -1;
            fa::prefill_work_item(m, w, qt, bh);
            plain_order(nwg, w, nq, g, c, qt0, bh0);
            if (qt != qt0 || bh != bh0) {
              std::printf("differs from the plain order: qtiles %d pairs %d group %d chunk %d w %d -> (%d, %d), "
                          "expected (%d, %d)\n", nq, np, g, c, w, qt, bh, qt0, bh0);
              return 1;
            }
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
