// Overflow guards of the sliced layouts: plain integer arithmetic (no HIP),
// so the host tests can compile and check them on their own.
#pragma once

#include <cstdint>

namespace sla {

constexpr int64_t kInt32Max = 2147483647;

// Slot offsets of a sliced layout are int32 (prefix sums over the slices and
// indices inside the kernels).  A layout of `nslices` slices whose widest
// slice has `max_width` slots of `lanes` entries each, plus `tail` padding
// entries, is representable when its largest possible size,
// nslices * max_width * lanes + tail, is below INT32_MAX.
constexpr bool sliced_layout_fits(int64_t nslices, int64_t max_width, int64_t lanes,
                                  int64_t tail) {
  if (nslices < 0 || max_width < 0 || lanes <= 0 || tail < 0 || tail >= kInt32Max) return false;
  if (nslices == 0 || max_width == 0) return true;
  const int64_t room = kInt32Max - 1 - tail;  // largest admissible nslices * max_width * lanes
  return max_width <= room / lanes && nslices <= room / (max_width * lanes);
}

}  // namespace sla
