// Gather (store) and scatter (retrieve) kernels for CDNA4 (gfx950).
//
// The work of a call is a flat list of tiles: every (chunk, layer, block j,
// tile s) is one span of at most tile_bytes contiguous bytes on both sides,
// because a page is contiguous in the pool (vLLM hybrid KV-cache blog,
// sections 3.1 and 3.2: a layer's page sits at offset + block_id * stride)
// and in the object.  One workgroup takes one tile:
//   - the tile's table entries (work item, layer placement, block id, object
//     address) are uniform across the workgroup and are read through the
//     constant address space, so they land in SGPRs (scalar loads);
//   - the bytes move as 16-byte vectors per lane, a wave covering 1 KiB
//     contiguous, with nontemporal hints (the pools are far larger than the
//     caches and nothing is reused);
//   - workgroups go round-robin over the 8 XCDs, so the item index is remapped
//     to give each XCD one contiguous range of tiles: at any moment the
//     workgroups of an XCD sweep a narrow window of a few pages instead of
//     striding across the whole batch;
//   - tiles are small (4 KiB by default) so that a window stays narrow: on
//     MI355X this measured best for both directions (about 6.9 TB/s of HBM
//     traffic for the gather and 6.3 TB/s for the scatter at the Kimi-Linear
//     TP=1 shapes, against 6.1 and 5.2 TB/s with 256 KiB tiles and no remap);
//   - only real page bytes are touched, so KDA padding (path A) and group
//     slack (path B) are never read or written.
// A page is opaque bytes ("Kimi-Linear" recipe: the KDA state is an opaque
// page), so data only ever lives in integer vector registers: NaN payloads
// of bf16/fp8 values pass unchanged.
#include <hip/hip_runtime.h>

#include "hkv_device_tables.hpp"
#include "hkv_launch.hpp"

#define HKV_GLOBAL __attribute__((address_space(1)))
#define HKV_CONST __attribute__((address_space(4)))

namespace {

// Build-time choices (defaults are the tuned ones).
#ifndef HKV_UNROLL
#define HKV_UNROLL 1      // 16-byte loads per lane issued before their stores
#endif
#ifndef HKV_NT_LOAD
#define HKV_NT_LOAD 1     // nontemporal loads
#endif
#ifndef HKV_NT_STORE
#define HKV_NT_STORE 1    // nontemporal stores
#endif
#ifndef HKV_XCD_REMAP
#define HKV_XCD_REMAP 1   // give each XCD a contiguous range of work items
#endif

constexpr uint32_t kThreads = hkv::kCopyThreads;
constexpr uint32_t kUnroll = HKV_UNROLL;
constexpr uint32_t kXcds = 8;  // MI355X: workgroups go round-robin over 8 XCDs

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u load16(const HKV_GLOBAL v4u* p) {
#if HKV_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ void store16(HKV_GLOBAL v4u* p, v4u v) {
#if HKV_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Copies `bytes` bytes from src to dst with all kThreads lanes of the
// workgroup.  Spans whose pointers and length are 16-byte multiples take the
// vector path; anything else (pages whose size is not a 16-byte multiple)
// falls back to byte copies.
__device__ __forceinline__ void copy_span(uint8_t* dst, const uint8_t* src, uint32_t bytes) {
  const uint32_t t = threadIdx.x;
  if (((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | bytes) & 15u) ==
      0) {
    const HKV_GLOBAL v4u* s = (const HKV_GLOBAL v4u*)src;
    HKV_GLOBAL v4u* d = (HKV_GLOBAL v4u*)dst;
    const uint32_t n = bytes >> 4;
    constexpr uint32_t kStep = kThreads * kUnroll;
    uint32_t base = 0;
    for (; base + kStep <= n; base += kStep) {
      v4u v[kUnroll];
#pragma unroll
      for (uint32_t u = 0; u < kUnroll; ++u) v[u] = load16(s + base + u * kThreads + t);
#pragma unroll
      for (uint32_t u = 0; u < kUnroll; ++u) store16(d + base + u * kThreads + t, v[u]);
    }
    for (uint32_t i = base + t; i < n; i += kThreads) store16(d + i, load16(s + i));
  } else {
    const HKV_GLOBAL uint8_t* s = (const HKV_GLOBAL uint8_t*)src;
    HKV_GLOBAL uint8_t* d = (HKV_GLOBAL uint8_t*)dst;
    for (uint32_t i = t; i < bytes; i += kThreads) d[i] = s[i];
  }
}

// Writes `bytes` zero bytes at dst with all kThreads lanes of the workgroup.
__device__ __forceinline__ void zero_span(uint8_t* dst, uint32_t bytes) {
  const uint32_t t = threadIdx.x;
  if (((reinterpret_cast<uintptr_t>(dst) | bytes) & 15u) == 0) {
    HKV_GLOBAL v4u* d = (HKV_GLOBAL v4u*)dst;
    const v4u z = {0u, 0u, 0u, 0u};
    for (uint32_t i = t; i < (bytes >> 4); i += kThreads) store16(d + i, z);
  } else {
    HKV_GLOBAL uint8_t* d = (HKV_GLOBAL uint8_t*)dst;
    for (uint32_t i = t; i < bytes; i += kThreads) d[i] = 0;
  }
}

template <bool kStore>
__device__ __forceinline__ void copy_items(const hkv::CopyArgs& a) {
  const HKV_CONST hkv::DevLayer* layers = (const HKV_CONST hkv::DevLayer*)a.layers;
  const HKV_CONST uint64_t* items = (const HKV_CONST uint64_t*)a.items;
  const HKV_CONST int32_t* ids = (const HKV_CONST int32_t*)a.ids;
  const HKV_CONST uint64_t* objs = (const HKV_CONST uint64_t*)a.objs;
  const uint32_t total = (uint32_t)a.total_items;
#if HKV_XCD_REMAP
  // Workgroup b runs on XCD b % 8; give XCD x the contiguous item range
  // [x*q + min(x, r), ...) of this round so one XCD works through whole pages.
  const uint32_t q = gridDim.x / kXcds, r = gridDim.x % kXcds;
  const uint32_t x = blockIdx.x % kXcds;
  const uint32_t first = x * q + (x < r ? x : r) + blockIdx.x / kXcds;
#else
  const uint32_t first = blockIdx.x;
#endif
  for (uint32_t item = first; item < total; item += gridDim.x) {
    const uint32_t c = item / a.items_per_chunk;
    const uint32_t r = item - c * a.items_per_chunk;
    const uint64_t w = items[r];
    const uint32_t l = (uint32_t)(w & 0xFFFFu);
    const uint32_t j = (uint32_t)((w >> 16) & 0xFFFFu);
    const uint32_t s = (uint32_t)(w >> 32);
    const HKV_CONST hkv::DevLayer* L = layers + l;
    const uint64_t page_bytes = L->page;
    const int32_t id = ids[((uint64_t)c * a.n_kv_groups + L->kv_group) * a.blocks_per_chunk + j];
    uint8_t* obj = reinterpret_cast<uint8_t*>(objs[(uint64_t)c * a.n_obj_groups + L->obj_group]);
    const uint64_t off = (uint64_t)s * a.tile_bytes;
    const uint64_t rest = page_bytes - off;
    const uint32_t bytes = (uint32_t)(rest < a.tile_bytes ? rest : a.tile_bytes);
    uint8_t* obj_tile = obj + L->obj_offset + (uint64_t)j * page_bytes + off;
    // Bytes of this page that hold data: all of it, none for a null id, and
    // for an MLA page of a partial chunk the rows of its valid tokens.
    uint64_t valid = id < 0 ? 0 : page_bytes;
    if (a.chunk_tokens && L->row_bytes && id >= 0) {
      int64_t rows = (int64_t)a.chunk_tokens[c] - (int64_t)j * (int64_t)a.block_tokens;
      rows = rows < 0 ? 0 : (rows > (int64_t)a.block_tokens ? (int64_t)a.block_tokens : rows);
      valid = (uint64_t)rows * L->row_bytes;
    }
    const uint32_t live =
        valid > off ? (uint32_t)(valid - off < bytes ? valid - off : bytes) : 0u;
    if (live) {
      uint8_t* page = a.pool + L->pool_offset + (uint64_t)id * L->stride + off;
      if (kStore)
        copy_span(obj_tile, page, live);
      else
        copy_span(page, obj_tile, live);
    }
    if (kStore && live < bytes) zero_span(obj_tile + live, bytes - live);
  }
}

}  // namespace

extern "C" __global__ __launch_bounds__(kThreads) void hkv_store_gather(hkv::CopyArgs a) {
  copy_items<true>(a);
}

extern "C" __global__ __launch_bounds__(kThreads) void hkv_retrieve_scatter(hkv::CopyArgs a) {
  copy_items<false>(a);
}

namespace hkv {

int launch_copy(bool store, const CopyArgs& a, uint32_t grid, void* stream) {
  if (grid == 0) return 0;
  CopyArgs arg = a;
  void* params[] = {&arg};
  const void* fn = store ? reinterpret_cast<const void*>(&hkv_store_gather)
                         : reinterpret_cast<const void*>(&hkv_retrieve_scatter);
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(kThreads), params, 0,
                              reinterpret_cast<hipStream_t>(stream));
}

}  // namespace hkv
