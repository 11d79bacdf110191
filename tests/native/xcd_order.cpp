// The work-item order of the copy kernels (hkv::xcd_first_item, shared with
// the kernels): for every run length and grid size, workgroups 0..grid-1 take
// distinct first items that cover [0, grid) -- a bijection, so every work
// item of a launch is processed exactly once (later rounds add multiples of
// grid).
#include <cstdio>
#include <vector>

#include "hkv_device_tables.hpp"

int main() {
  const uint32_t kXcds = 8;
  for (uint32_t run : {0u, 1u, 7u, 64u, 530u, 8192u}) {
    for (uint32_t grid : {1u, 7u, 8u, 9u, 63u, 64u, 65u, 511u, 512u, 4239u, 65537u, 100003u,
                          14660608u}) {
      std::vector<uint8_t> seen(grid, 0);
      for (uint32_t b = 0; b < grid; ++b) {
        const uint32_t first = hkv::xcd_first_item(b, grid, run, kXcds);
        if (first >= grid || seen[first]) {
          std::printf("run %u grid %u: workgroup %u takes item %u twice or out of range\n", run,
                      grid, b, first);
          return 1;
        }
        seen[first] = 1;
      }
    }
  }
  std::printf("xcd order: bijection for every run length and grid size\n");
  return 0;
}
