// Host-only driver for the launch-size arithmetic of the pair kernels
// (launch_plan.h): reads "nrows ncols slots d" lines on stdin and prints the
// planned split "G glog cps nchunks tiles ok" for the dense VALU kernel with
// its constants (16-column chunks, 128-row tiles, 8 waves of 64, at most 64
// splits, 8 XCDs, 2 MiB of column data per XCD L2).
#include <cstdio>

#include "launch_plan.h"

int main() {
  long long nrows, ncols, slots;
  int d;
  std::printf("max_blocks_512 %lld\n", (long long)sk::max_blocks_1d(512));
  while (std::scanf("%lld %lld %lld %d", &nrows, &ncols, &slots, &d) == 4) {
    const sk::DenseSplit s =
        sk::plan_dense_split(nrows, ncols, slots, d, 16, 128, 8, 512, 64, 8, 2 << 20);
    std::printf("%d %d %lld %lld %lld %d\n", s.G, s.glog, (long long)s.cps, (long long)s.nchunks,
                (long long)s.tiles, s.ok ? 1 : 0);
  }
  return 0;
}
