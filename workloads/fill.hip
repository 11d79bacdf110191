// Counter-based SplitMix64 fill of device memory: word q of a buffer with
// seed s is mix64(s + (word0 + q + 1) * GAMMA), stored little-endian.
// This is input generation for tests and benchmarks (the same definition as
// workloads/__init__.py), not part of the store/retrieve library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void splitmix_fill_words(uint64_t* __restrict__ dst,
                                                           uint64_t n_words, uint64_t seed,
                                                           uint64_t word0) {
  const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n_words; q += step)
    dst[q] = mix64(seed + (word0 + q + 1) * kGamma);
}

// The last partial word: bytes [0, n_tail) of word `q` go to dst[0..n_tail).
__global__ void splitmix_fill_tail(uint8_t* __restrict__ dst, uint32_t n_tail, uint64_t seed,
                                   uint64_t q) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const uint64_t w = mix64(seed + (q + 1) * kGamma);
    for (uint32_t b = 0; b < n_tail; ++b) dst[b] = (uint8_t)(w >> (8 * b));
  }
}

}  // namespace

// Returns 0 or the hipError_t value.  dst must be 8-byte aligned.
extern "C" int hkvfill_splitmix(void* dst, uint64_t nbytes, uint64_t seed, uint64_t word0,
                                void* stream) {
  if (nbytes == 0) return 0;
  if (reinterpret_cast<uintptr_t>(dst) & 7) return (int)hipErrorInvalidValue;
  // The launch statuses are returned directly: hipGetLastError() would also
  // report an earlier failure of any other HIP call on this thread.
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint64_t n_words = nbytes / 8;
  const uint32_t n_tail = (uint32_t)(nbytes % 8);
  if (n_words) {
    uint64_t blocks = (n_words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    uint64_t* words = reinterpret_cast<uint64_t*>(dst);
    void* args[] = {&words, const_cast<uint64_t*>(&n_words), &seed, &word0};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&splitmix_fill_words),
                                         dim3((uint32_t)blocks), dim3(256), args, 0, s);
    if (e != hipSuccess) return (int)e;
  }
  if (n_tail) {
    uint8_t* tail = reinterpret_cast<uint8_t*>(dst) + n_words * 8;
    uint64_t q = word0 + n_words;
    uint32_t nt = n_tail;
    void* args[] = {&tail, &nt, &seed, &q};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&splitmix_fill_tail),
                                         dim3(1), dim3(64), args, 0, s);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}
