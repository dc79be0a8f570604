// Host check of the decode kernel's workgroup ranges (pkv_internal.h): for a sweep of batch sizes,
// workgroup counts and odd-XCD weights, the ranges tile [0, W) in order, range_owner is the exact
// inverse of range_start at every range boundary, and the range <-> workgroup map is a bijection
// that gives XCD x (workgroups w with w % 8 == x) the consecutive ranges [x P, (x + 1) P) when the
// workgroup count is a multiple of 8. The split-stream merge relies on this: every part of a
// stream must name the same first range and the same number of parts.
#include "pkv_internal.h"

#include <cstdio>
#include <vector>

int main() {
  using namespace pkv;
  const int Ws[] = {1, 2, 3, 7, 64, 100, 511, 512, 513, 1000, 45168, 131072, 151552, 1 << 20,
                    (1 << 27) + 12345, 2147483647};
  const int nwgs[] = {1, 2, 3, 7, 8, 9, 16, 64, 255, 256, 500, 512, 2000, 2048, 4096, 1 << 20};
  const int weights[] = {kEvenWeight, 900, kEvenWeight / 2, 777};
  long long checked = 0, bad = 0;
  for (int nwg : nwgs) {
    std::vector<char> seen(nwg, 0);
    const int nx = range_blocks(nwg), per = nwg / nx;
    for (int w = 0; w < nwg; ++w) {
      const int r = range_of_workgroup(w, nwg);
      if (r < 0 || r >= nwg || seen[r] || workgroup_of_range(r, nwg) != w ||
          (nx == 8 && r / per != w % 8)) {
        if (bad++ < 10) printf("map nwg=%d w=%d r=%d\n", nwg, w, r);
        continue;
      }
      seen[r] = 1;
    }
  }
  for (int W : Ws) {
    for (int nwg0 : nwgs) {
      const int nwg = nwg0 < W ? nwg0 : W;
      for (int ow : weights) {
        if (range_start(0, nwg, W, ow) != 0 || range_start(nwg, nwg, W, ow) != W) {
          if (bad++ < 10) printf("ends W=%d nwg=%d ow=%d\n", W, nwg, ow);
        }
        const int stride = nwg > 4096 ? 61 : 1;
        for (int r = 0; r < nwg; r += (r + stride < nwg ? stride : 1)) {
          const int a = range_start(r, nwg, W, ow), b = range_start(r + 1, nwg, W, ow);
          ++checked;
          if (b < a) {
            if (bad++ < 10) printf("order W=%d nwg=%d ow=%d r=%d\n", W, nwg, ow, r);
            continue;
          }
          if (b > a && (range_owner(a, nwg, W, ow) != r || range_owner(b - 1, nwg, W, ow) != r)) {
            if (bad++ < 10) printf("owner W=%d nwg=%d ow=%d r=%d\n", W, nwg, ow, r);
          }
          // with weights of at least half the even weight and W >= 2 nwg, no range is empty
          if (W >= 2 * nwg && b == a) {
            if (bad++ < 10) printf("empty W=%d nwg=%d ow=%d r=%d\n", W, nwg, ow, r);
          }
        }
        // every position of a sample belongs to the range range_owner names
        const long long step = W > 100000 ? W / 9973 + 1 : 1;
        for (long long p = 0; p < W; p += step) {
          const int r = range_owner((int)p, nwg, W, ow);
          if (!(range_start(r, nwg, W, ow) <= p && p < range_start(r + 1, nwg, W, ow))) {
            if (bad++ < 10) printf("member W=%d nwg=%d ow=%d p=%lld\n", W, nwg, ow, p);
          }
        }
      }
    }
  }
  // plan_ranges: never more workgroups than the grid or the positions, at least one when there
  // are positions; the full count unless may_halve, else the full count or its half; an aligned
  // plan cuts W into equal ranges of whole L-unit streams and weighs nothing; weights only where
  // every range keeps a position.
  const int Ls[] = {0, 1, 3, 16, 64, 256, 512};
  const int grids[] = {1, 2, 7, 8, 64, 128, 256, 512, 1024};
  for (int L : Ls) {
    for (int streams : {1, 7, 64, 256, 512, 513, 1280, 4096}) {
      const long long Wl = (long long)streams * (L > 0 ? L : 37);
      if (Wl >= 2147483647LL) continue;
      const int W = (int)Wl;
      for (int grid : grids) {
        for (int halve = 0; halve < 2; ++halve) {
          const RangePlan p = plan_ranges(W, L, grid, halve != 0, 900);
          const int full = grid < W ? grid : W;
          ++checked;
          bool ok = p.nwg >= 1 && p.nwg <= full;
          ok = ok && (halve ? (p.nwg == full || p.nwg == full / 2) : p.nwg == full);
          if (p.aligned)
            ok = ok && L > 0 && W % p.nwg == 0 && (W / p.nwg) % L == 0 && p.odd_w == kEvenWeight;
          if (p.odd_w != kEvenWeight) ok = ok && !p.aligned && W >= 2 * p.nwg;
          if (!ok && bad++ < 10)
            printf("plan W=%d L=%d grid=%d halve=%d -> nwg=%d odd_w=%d aligned=%d\n", W, L, grid,
                   halve, p.nwg, p.odd_w, (int)p.aligned);
        }
      }
    }
  }
  printf("ranges checked %lld, failures %lld\n", checked, bad);
  return bad ? 1 : 0;
}
