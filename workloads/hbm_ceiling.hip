// HBM reference rates for the roofline context of the copy kernels: a pure
// read, a pure write and a contiguous buffer-to-buffer copy, each with the
// same structure as the library's kernels (one 4 KiB tile per 128-thread
// workgroup, tiles in XCD order, 16-byte nontemporal accesses).  Measurement
// harness only; not part of the store/retrieve library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#define HKV_GLOBAL __attribute__((address_space(1)))
constexpr uint32_t kThreads = 128;
constexpr uint32_t kTileVec = 4096 / 16;

__device__ __forceinline__ uint32_t xcd_tile() {
  const uint32_t q = gridDim.x / 8, r = gridDim.x % 8, x = blockIdx.x % 8;
  return x * q + (x < r ? x : r) + blockIdx.x / 8;
}

__global__ __launch_bounds__(kThreads) void ceiling_read(const v4u* src, uint32_t* out,
                                                         uint32_t n_tiles) {
  const uint32_t tile = xcd_tile();
  if (tile >= n_tiles) return;
  const HKV_GLOBAL v4u* s = (const HKV_GLOBAL v4u*)(src + (uint64_t)tile * kTileVec);
  uint32_t acc = 0;
  for (uint32_t i = threadIdx.x; i < kTileVec; i += kThreads) {
    const v4u v = __builtin_nontemporal_load(s + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[tile] = acc;  // keeps the loads; almost never stores
}

__global__ __launch_bounds__(kThreads) void ceiling_write(v4u* dst, uint32_t n_tiles) {
  const uint32_t tile = xcd_tile();
  if (tile >= n_tiles) return;
  HKV_GLOBAL v4u* d = (HKV_GLOBAL v4u*)(dst + (uint64_t)tile * kTileVec);
  const v4u v = {tile, threadIdx.x, 0x5Au, 0xA5u};
  for (uint32_t i = threadIdx.x; i < kTileVec; i += kThreads) __builtin_nontemporal_store(v, d + i);
}

__global__ __launch_bounds__(kThreads) void ceiling_copy(const v4u* src, v4u* dst,
                                                         uint32_t n_tiles) {
  const uint32_t tile = xcd_tile();
  if (tile >= n_tiles) return;
  const HKV_GLOBAL v4u* s = (const HKV_GLOBAL v4u*)(src + (uint64_t)tile * kTileVec);
  HKV_GLOBAL v4u* d = (HKV_GLOBAL v4u*)(dst + (uint64_t)tile * kTileVec);
  for (uint32_t i = threadIdx.x; i < kTileVec; i += kThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

}  // namespace

// kind 0 = read src, 1 = write dst, 2 = copy src -> dst.  bytes must be a
// multiple of 4096 and below 2^44; out needs bytes / 4096 words (read only).
// Returns the hipError_t of the launch.
extern "C" int hkvceiling_launch(int kind, const void* src, void* dst, void* out, uint64_t bytes,
                                 void* stream) {
  if (bytes % 4096 || bytes / 4096 > 0xFFFFFFFFull / kThreads) return (int)hipErrorInvalidValue;
  uint32_t n_tiles = (uint32_t)(bytes / 4096);
  if (n_tiles == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const v4u* sv = static_cast<const v4u*>(src);
  v4u* dv = static_cast<v4u*>(dst);
  uint32_t* ov = static_cast<uint32_t*>(out);
  void* args_read[] = {&sv, &ov, &n_tiles};
  void* args_write[] = {&dv, &n_tiles};
  void* args_copy[] = {&sv, &dv, &n_tiles};
  const void* fn = kind == 0 ? reinterpret_cast<const void*>(&ceiling_read)
                 : kind == 1 ? reinterpret_cast<const void*>(&ceiling_write)
                             : reinterpret_cast<const void*>(&ceiling_copy);
  void** args = kind == 0 ? args_read : kind == 1 ? args_write : args_copy;
  if (kind < 0 || kind > 2) return (int)hipErrorInvalidValue;
  return (int)hipLaunchKernel(fn, dim3(n_tiles), dim3(kThreads), args, 0, s);
}
