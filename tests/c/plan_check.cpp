// Host check of the matrix-core walk's launch shape (gated_delta_rule_59_amd/csrc/kda_plan.h),
// compiled with g++ and run on the CPU. Prints "ok" and returns 0 when every case holds.
#include <cstdio>

#include "kda_plan.h"

static int failures = 0;

static void expect(bool c, const char* what) {
  if (!c) {
    std::printf("FAIL: %s\n", what);
    ++failures;
  }
}

int main() {
  using kda::walk_shape;
  // 16 heads of one sequence on 256 CUs: 128 one-strip walks, two workgroups each
  expect(walk_shape(16, 256, false).strips == 1, "16 pairs: one strip per workgroup");
  expect(walk_shape(16, 256, false).halves == 2, "16 pairs: two workgroups per walk");
  // in place, the second workgroup could read a final state the first already stored
  expect(walk_shape(16, 256, true).halves == 1, "16 pairs in place: one workgroup per walk");
  // 32 heads: 256 strips, two per workgroup, 128 walks, still two workgroups each
  expect(walk_shape(32, 256, false).strips == 2, "32 pairs: two strips per workgroup");
  expect(walk_shape(32, 256, false).halves == 2, "32 pairs: two workgroups per walk");
  expect(walk_shape(32, 256, true).halves == 1, "32 pairs in place: one workgroup per walk");
  // 512 pairs fill the chip without repeating the walk, four strips per workgroup
  expect(walk_shape(512, 256, false).halves == 1, "512 pairs: one workgroup per walk");
  expect(walk_shape(512, 256, false).strips == 4, "512 pairs: four strips per workgroup");
  // the thresholds: four strips from 128 pairs (1,024 strips) on 256 CUs, two below
  expect(walk_shape(128, 256, false).strips == 4 && walk_shape(128, 256, false).halves == 1,
         "128 pairs: four strips, one workgroup per walk");
  expect(walk_shape(127, 256, false).strips == 2 && walk_shape(127, 256, false).halves == 1,
         "127 pairs: two strips, one workgroup per walk");
  expect(walk_shape(31, 256, false).strips == 1 && walk_shape(31, 256, false).halves == 1,
         "31 pairs: one strip, one workgroup per walk");
  // one pair: eight strips, two workgroups each
  expect(walk_shape(1, 256, false).halves == 2 && walk_shape(1, 256, false).strips == 1,
         "1 pair");
  expect(walk_shape(1, 256, true).halves == 1, "1 pair in place");
  if (failures == 0) std::printf("ok\n");
  return failures ? 1 : 0;
}
