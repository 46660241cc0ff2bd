// Grouped calls: consecutive row slices of one input, each quantized as a
// tensor of its own (one amax per group, its own data and scale blocks).
// The table travels in the kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr uint32_t kMaxGroups = 256;

struct GroupTable {
  uint32_t ngroups;
  uint32_t row_start[kMaxGroups + 1];   // first input row of group g; [ngroups] = total rows
  uint32_t unit_start[kMaxGroups + 1];  // first work unit (tile, chunk) of group g; [ngroups] = total units
  uint32_t part_start[kMaxGroups + 1];  // first workspace maximum of group g (multiples of 4)
};

// The group that owns work unit `unit` (< unit_start[ngroups]): the g with
// unit_start[g] <= unit < unit_start[g + 1], which skips empty groups.
// Uniform (a scalar binary search over the kernel arguments).
__device__ __forceinline__ uint32_t group_of(const GroupTable &t, uint32_t unit) {
  uint32_t lo = 0, hi = t.ngroups;  // unit_start[lo] <= unit < unit_start[hi]
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (t.unit_start[mid] <= unit)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

}  // namespace nvfp4
