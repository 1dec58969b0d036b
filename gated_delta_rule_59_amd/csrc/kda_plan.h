// Launch-shape choices of the matrix-core prefill walk, as plain host arithmetic with no HIP
// types, so that they can be checked on a machine without a GPU.
#pragma once

#include <stdint.h>

namespace kda {

struct WalkShape {
  int strips;  // 16-column strips of the state a workgroup carries: 1, 2 or 4
  int halves;  // workgroups per walk: 2 = two workgroups repeat the same state walk and each
               // writes the outputs of half of the chunk rows
};

// pairs: (sequence, head) pairs; n_cu: compute units; in_place: S_T is the S0 buffer.
//  - From one 16-column strip per CU on, two strips per workgroup halve the state operand
//    bytes per column (the walk is bound by each CU's vector memory unit); from four strips
//    per CU on, four per workgroup quarter them (varlen-16, 512 pairs: -2.3 %), while fewer
//    would leave CUs idle (prefill-64k-bound, 32 pairs, at four strips: +17 %).
//  - When the walks would leave at least half of the CUs idle, two workgroups per walk repeat
//    the state walk and split the output rows. Both read S0 when they start and only the first
//    writes S_T when it ends, which is correct only while S0 is not written during the launch:
//    when S_T is the S0 buffer the second workgroup could start after the first has already
//    stored the final state, so an in-place call always walks with one workgroup.
inline WalkShape walk_shape(int64_t pairs, int n_cu, bool in_place) {
  constexpr int64_t kStrips = 8;  // 16-column strips of a 128-column state
  WalkShape s;
  const int64_t all = pairs * kStrips;
  s.strips = all >= 4 * (int64_t)n_cu ? 4 : all >= (int64_t)n_cu ? 2 : 1;
  const int64_t walks = all / s.strips;
  s.halves = (!in_place && walks * 2 <= (int64_t)n_cu) ? 2 : 1;
  return s;
}

}  // namespace kda
