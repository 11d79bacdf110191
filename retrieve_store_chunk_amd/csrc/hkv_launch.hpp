// Host-side entry to the copy kernels.
#pragma once

#include <cstdint>

#include "hkv_device_tables.hpp"

namespace hkv {

#ifndef HKV_THREADS
#define HKV_THREADS 128  // two waves per workgroup
#endif
constexpr uint32_t kCopyThreads = HKV_THREADS;

// Enqueues the gather (store) or scatter (retrieve) kernel over
// a.total_items work items with `grid` workgroups on `stream` (a
// hipStream_t); `t` carries the per-call tables that a leaves null.
// Returns the hipError_t of the launch (0 = success).
int launch_copy(bool store, const CopyArgs& a, const InlineTables& t, uint32_t grid,
                void* stream);

}  // namespace hkv
