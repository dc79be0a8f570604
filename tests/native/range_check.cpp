// Host check of the decode kernel's workgroup ranges (pkv_internal.h): for a sweep of batch sizes,
// workgroup counts and odd-XCD weights, the ranges tile [0, W) in order and range_owner is the
// exact inverse of range_start at every range boundary. The split-stream merge relies on this:
// every part of a stream must name the same first workgroup and the same number of parts.
#include "pkv_internal.h"

#include <cstdio>

int main() {
  using namespace pkv;
  const int Ws[] = {1, 2, 3, 7, 64, 100, 511, 512, 513, 1000, 45168, 131072, 151552, 1 << 20,
                    (1 << 27) + 12345, 2147483647};
  const int nwgs[] = {1, 2, 3, 7, 8, 9, 64, 255, 256, 500, 512, 2000, 4096, 1 << 20};
  const int weights[] = {kEvenWeight, 900, kEvenWeight / 2, 777};
  long long checked = 0, bad = 0;
  for (int W : Ws) {
    for (int nwg0 : nwgs) {
      const int nwg = nwg0 < W ? nwg0 : W;
      for (int ow : weights) {
        if (range_start(0, nwg, W, ow) != 0 || range_start(nwg, nwg, W, ow) != W) {
          if (bad++ < 10) printf("ends W=%d nwg=%d ow=%d\n", W, nwg, ow);
        }
        const int stride = nwg > 4096 ? 61 : 1;
        for (int w = 0; w < nwg; w += (w + stride < nwg ? stride : 1)) {
          const int a = range_start(w, nwg, W, ow), b = range_start(w + 1, nwg, W, ow);
          ++checked;
          if (b < a) {
            if (bad++ < 10) printf("order W=%d nwg=%d ow=%d w=%d\n", W, nwg, ow, w);
            continue;
          }
          if (b > a && (range_owner(a, nwg, W, ow) != w || range_owner(b - 1, nwg, W, ow) != w)) {
            if (bad++ < 10) printf("owner W=%d nwg=%d ow=%d w=%d\n", W, nwg, ow, w);
          }
          // with weights of at least half the even weight and W >= 2 nwg, no range is empty
          if (W >= 2 * nwg && b == a) {
            if (bad++ < 10) printf("empty W=%d nwg=%d ow=%d w=%d\n", W, nwg, ow, w);
          }
        }
      }
    }
  }
  printf("ranges checked %lld, failures %lld\n", checked, bad);
  return bad ? 1 : 0;
}
