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

// Rows of streams at given places in one buffer.  Row r is four words:
// byte offset (a multiple of 8) into the buffer, seed, first word index, and
// word count, whose top bit asks for zeros instead of stream words.
// Workgroup b writes tile b % tiles_per_row of row b / tiles_per_row.  A row
// that would end past buf_bytes is not written at all.
__global__ __launch_bounds__(256) void splitmix_fill_rows(uint8_t* __restrict__ base,
                                                          uint64_t buf_bytes,
                                                          const uint64_t* __restrict__ rows,
                                                          uint64_t n_rows, uint32_t tiles_per_row,
                                                          uint32_t tile_words) {
  const uint64_t row = blockIdx.x / tiles_per_row;
  const uint64_t tile = blockIdx.x % tiles_per_row;
  if (row >= n_rows) return;
  const uint64_t off = rows[4 * row], seed = rows[4 * row + 1], word0 = rows[4 * row + 2];
  const uint64_t count = rows[4 * row + 3];
  const uint64_t n_words = count & ~(1ull << 63);
  const bool zeros = (count >> 63) != 0;
  if ((off & 7) || off > buf_bytes || n_words > (buf_bytes - off) / 8) return;
  const uint64_t lo = tile * tile_words;
  if (lo >= n_words) return;
  const uint64_t hi = lo + tile_words < n_words ? lo + tile_words : n_words;
  uint64_t* d = reinterpret_cast<uint64_t*>(base + off);
  for (uint64_t q = lo + threadIdx.x; q < hi; q += blockDim.x)
    d[q] = zeros ? 0ull : mix64(seed + (word0 + q + 1) * kGamma);
}

}  // namespace

// Rows (see splitmix_fill_rows) from a DEVICE table of n_rows x 4 words into
// the buffer at base (8-byte aligned, buf_bytes long); max_words bounds every
// row's word count.  Returns 0 or the hipError_t value.
extern "C" int hkvfill_rows(void* base, uint64_t buf_bytes, const void* rows, uint64_t n_rows,
                            uint64_t max_words, void* stream) {
  if (n_rows == 0 || max_words == 0) return 0;
  if (reinterpret_cast<uintptr_t>(base) & 7) return (int)hipErrorInvalidValue;
  constexpr uint32_t kTileWords = 8192;  // 64 KiB per workgroup
  const uint64_t tiles = (max_words + kTileWords - 1) / kTileWords;
  const uint64_t grid = n_rows * tiles;
  if (grid > 0xFFFFFFFFull / 256) return (int)hipErrorInvalidValue;  // 32-bit work-item count
  uint8_t* b = static_cast<uint8_t*>(base);
  const uint64_t* r = static_cast<const uint64_t*>(rows);
  uint32_t tpr = (uint32_t)tiles, tw = kTileWords;
  void* args[] = {&b, &buf_bytes, &r, &n_rows, &tpr, &tw};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&splitmix_fill_rows),
                              dim3((uint32_t)grid), dim3(256), args, 0,
                              reinterpret_cast<hipStream_t>(stream));
}

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
