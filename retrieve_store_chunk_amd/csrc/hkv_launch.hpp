// Host-side entry to the copy kernels.
#pragma once

#include <cstdint>

#include "hkv_device_tables.hpp"

namespace hkv {

constexpr uint32_t kCopyThreads = 128;  // two waves per workgroup

// Enqueues the gather (store) or scatter (retrieve) kernel over
// a.total_items work items with `grid` workgroups on `stream` (a
// hipStream_t); `t` carries the per-call tables that a leaves null.
// Returns the hipError_t of the launch (0 = success).
int launch_copy(bool store, const CopyArgs& a, const InlineTables& t, uint32_t grid,
                void* stream);

// Bytes of the static device array that hkv_move_chunks_noalloc keeps a
// layout's tables in (one copy per device, held until the process ends).
constexpr uint64_t kStaticScratchBytes = uint64_t(4) << 20;

// The device address of that array on device `dev`, which must be the
// current device: looked up once per device, then remembered.  Returns the
// hipError_t of the lookup (0 = success).
int static_scratch(int dev, uint8_t** ptr);

}  // namespace hkv
