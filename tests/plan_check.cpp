// Host checks of the workgroup-to-XCD order in csrc/ra_plan.h (built and run
// by tests/test_plan_native.py with the host compiler).
#include "ra_plan.h"

#include <cstdio>
#include <vector>

int main() {
  // a bijection on [0, nwg) for every grid and run length
  for (int nwg : {1, 7, 8, 16, 24, 64, 256, 512, 1000, 1024, 2048, 8192})
    for (int run : {1, 3, 16, 32, 64, 96, 128, 256, 1024, 4096}) {
      std::vector<int> seen(nwg, 0);
      for (int b = 0; b < nwg; ++b) {
        const int l = ra_plan_xcd_remap(b, nwg, run);
        if (l < 0 || l >= nwg) { std::printf("out of range: nwg %d run %d\n", nwg, run); return 1; }
        ++seen[l];
      }
      for (int v : seen)
        if (v != 1) { std::printf("not a bijection: nwg %d run %d\n", nwg, run); return 1; }
    }
  // causal work per XCD (query tile t of a head has t + 1 units, later tiles
  // first) within 2 % of the mean, and each XCD holds tiles of as few heads
  // as the grid allows
  struct Case { int nqt, heads; };
  for (Case c : {Case{256, 4}, Case{16, 32}, Case{32, 8}, Case{512, 2}, Case{1024, 1}}) {
    const int nwg = c.nqt * c.heads;
    double w[8] = {0};
    std::vector<std::vector<int>> heads(8);
    for (int b = 0; b < nwg; ++b) {
      const int l = ra_plan_xcd_remap(b, nwg, c.nqt), qt = c.nqt - 1 - l % c.nqt, h = l / c.nqt;
      w[b % 8] += qt + 1;
      bool have = false;
      for (int x : heads[b % 8]) have |= x == h;
      if (!have) heads[b % 8].push_back(h);
    }
    double mean = 0;
    for (double x : w) mean += x / 8;
    const int want = c.heads >= 8 ? c.heads / 8 : 1;
    for (int x = 0; x < 8; ++x) {
      if (w[x] > 1.02 * mean || w[x] < 0.98 * mean) {
        std::printf("unbalanced: nqt %d heads %d xcd %d work %g mean %g\n", c.nqt, c.heads, x, w[x], mean);
        return 1;
      }
      if ((int)heads[x].size() != want) {
        std::printf("xcd %d holds %zu heads (nqt %d heads %d)\n", x, heads[x].size(), c.nqt, c.heads);
        return 1;
      }
    }
  }
  // (head, query tile) of every workgroup: a bijection onto heads x tiles for
  // every grid, causal or not; when each XCD holds an even number of whole
  // heads, consecutive workgroups of an XCD alternate between two heads at the
  // same tile, later tiles first under causal masking
  for (int nqt : {1, 2, 3, 16, 32, 64, 256})
    for (int heads : {1, 2, 3, 4, 8, 16, 32, 64})
      for (int causal : {0, 1}) {
        const int nwg = nqt * heads;
        std::vector<int> seen(nwg, 0);
        for (int b = 0; b < nwg; ++b) {
          int h, t;
          ra_plan_head_tile(ra_plan_xcd_remap(b, nwg, nqt), nwg, nqt, causal, &h, &t);
          if (h < 0 || h >= heads || t < 0 || t >= nqt) {
            std::printf("head/tile out of range: nqt %d heads %d\n", nqt, heads);
            return 1;
          }
          ++seen[h * nqt + t];
        }
        for (int v : seen)
          if (v != 1) { std::printf("head/tile not a bijection: nqt %d heads %d\n", nqt, heads); return 1; }
      }
  {
    const int nqt = 16, heads = 32, nwg = nqt * heads;  // 4 heads per XCD
    for (int x = 0; x < 8; ++x)
      for (int i = 0; i + 1 < nwg / 8; i += 2) {
        int h0, t0, h1, t1;
        ra_plan_head_tile(ra_plan_xcd_remap(8 * i + x, nwg, nqt), nwg, nqt, 1, &h0, &t0);
        ra_plan_head_tile(ra_plan_xcd_remap(8 * (i + 1) + x, nwg, nqt), nwg, nqt, 1, &h1, &t1);
        if (h1 != h0 + 1 || t1 != t0 || t0 != nqt - 1 - (i / 2) % nqt) {
          std::printf("pair order broken: xcd %d slot %d\n", x, i);
          return 1;
        }
      }
  }
  // Dispatch of the rank-7-of-8 share (16 query tiles of 256 rows per head,
  // 32 heads; a tile t of the diagonal block costs 7 full blocks of 64 key
  // tiles plus 4 (t + 1) diagonal ones) on 8 XCDs of 32 CUs, one workgroup
  // per CU, each next workgroup of an XCD to the CU that frees up first: the
  // paired order gives every CU the same work (the makespan equals the mean
  // load), while one head's tiles in a row leave 3 % of it on the table.
  {
    const int nqt = 16, heads = 32, nwg = nqt * heads, cus = 32;
    double worst = 0, total = 0;
    for (int x = 0; x < 8; ++x) {
      std::vector<double> free_at(cus, 0.0);
      for (int i = 0; i < nwg / 8; ++i) {
        int h, t;
        ra_plan_head_tile(ra_plan_xcd_remap(8 * i + x, nwg, nqt), nwg, nqt, 1, &h, &t);
        const double cost = 7 * 64 + 4 * (t + 1);
        int best = 0;
        for (int c = 1; c < cus; ++c)
          if (free_at[c] < free_at[best]) best = c;
        free_at[best] += cost;
        total += cost;
      }
      for (double f : free_at) worst = f > worst ? f : worst;
    }
    const double mean = total / (8.0 * cus);
    if (worst > mean * 1.001) {
      std::printf("unbalanced dispatch: makespan %g, mean load %g\n", worst, mean);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}
