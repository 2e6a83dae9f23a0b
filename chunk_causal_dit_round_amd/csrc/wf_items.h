// Work-group -> work item of an attention launch, placed for L2 locality.
//
// A launch's work items are (run, head, query tile), runs longest first (a
// run is a query group, or half of a split one).  The query tiles of one
// (run, head) -- a unit -- all read the same keys and values.  MI355X
// dispatches work-group b of a launch to XCD b mod 8, and every XCD has an
// L2 of its own: if the work-groups of a unit are spread over all eight,
// every XCD fetches the unit's K/V beyond its L2.  Here each XCD gets whole
// units instead: units are dealt to the XCDs in rounds of eight, the order
// reversed every other round, so the launch stays longest first overall and
// the XCDs get equal work when unit lengths come in multiples of eight
// (the 1.3B round: 72 units, 9 per XCD).  Units past the last full round
// keep their place.  The mapping is a bijection whatever the device does, so
// only locality, never correctness, depends on the dispatch order.
#pragma once

#include <hip/hip_runtime.h>

namespace wf {

__device__ inline int xcd_item(int b, int n_items, int q_tiles) {
  const int n8 = (n_items / q_tiles) & ~7;        // units in full rounds of eight
  if (b >= n8 * q_tiles) return b;
  const int x = b & 7, k = b >> 3;                // XCD, its k-th work-group
  const int j = k / q_tiles, qt = k - j * q_tiles;
  const int u = 8 * j + ((j & 1) ? 7 - x : x);    // the round's unit for this XCD
  return u * q_tiles + qt;
}

}  // namespace wf
