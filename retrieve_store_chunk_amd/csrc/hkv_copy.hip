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
//     so that the workgroups of an XCD sweep a narrow window of a few pages
//     instead of striding across the whole batch.  The gather gives each XCD
//     one contiguous range of items; the scatter lets the XCDs take turns on
//     runs of 8192 items (32 MiB), so that they work on neighbouring pages;
//   - tiles are small (4 KiB by default) so that a window stays narrow; the
//     gather issues two 16-byte loads per lane before its stores, the
//     scatter one.  On MI355X these measured best per direction (about
//     6.9 TB/s of HBM traffic for the gather and 6.4 TB/s for the scatter at
//     the Kimi-Linear TP=1 shapes, against 6.1 and 5.2 TB/s with 256 KiB
//     tiles and no remap);
//   - only real page bytes are touched, so KDA padding (path A) and group
//     slack (path B) are never read or written;
//   - layouts without the INT8 codec run a kernel pair with no codec code;
//     INT8 layouts run the pair built for their head_dim, so that each
//     kernel holds only the registers its own path needs.  The plain
//     kernels are capped by an LDS reservation at launch at 12 (gather) and
//     13 (scatter) workgroups per CU, where they measured best; the INT8
//     gather runs best at 8 waves per SIMD, which its registers allow.
// A page is opaque bytes ("Kimi-Linear" recipe: the KDA state is an opaque
// page), so data only ever lives in integer vector registers: NaN payloads
// of bf16/fp8 values pass unchanged.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hkv_device_tables.hpp"
#include "hkv_launch.hpp"

// The no-allocation entry point's scratch: a layout's tables (layer
// placements, work items) live here instead of in memory the library
// allocates.  Host code never names it after the lookup in
// hkv::static_scratch: on the host the name is only a stand-in for the
// symbol, not a device address.
static __device__ __align__(256) uint8_t scratch[hkv::kStaticScratchBytes];

#define HKV_GLOBAL __attribute__((address_space(1)))
#define HKV_CONST __attribute__((address_space(4)))

namespace {

constexpr uint32_t kThreads = hkv::kCopyThreads;
constexpr uint32_t kXcds = 8;  // MI355X: workgroups go round-robin over 8 XCDs

// Per direction, as measured best on MI355X at the Kimi-Linear shapes:
// 16-byte loads per lane issued before their stores; how the XCDs share the
// items (0: each XCD one contiguous range; n: the XCDs take turns on runs of
// n items); and the LDS each plain workgroup reserves without using it, which
// caps a CU at 12 gather (160 KiB / 13 KiB) or 13 scatter workgroups.
constexpr uint32_t kStoreUnroll = 2;
constexpr uint32_t kRetrieveUnroll = 1;
constexpr uint32_t kStoreXcdRun = 0;
constexpr uint32_t kRetrieveXcdRun = 8192;
constexpr uint32_t kGatherLds = 13312;
constexpr uint32_t kScatterLds = 12288;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Every access is nontemporal: the pools are far larger than the caches and
// nothing is read twice.
__device__ __forceinline__ v4u load16(const HKV_GLOBAL v4u* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store16(HKV_GLOBAL v4u* p, v4u v) {
  __builtin_nontemporal_store(v, p);
}

// Copies `bytes` bytes from src to dst with all kThreads lanes of the
// workgroup.  Spans whose pointers and length are 16-byte multiples take the
// vector path; anything else (pages whose size is not a 16-byte multiple)
// falls back to byte copies.
template <uint32_t kUnroll>
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

__device__ __forceinline__ uint32_t load4(const HKV_GLOBAL uint32_t* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store4(HKV_GLOBAL uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// kVecs consecutive 4-byte words at p (aligned to their total width).
template <uint32_t kVecs>
__device__ __forceinline__ void store_words(HKV_GLOBAL uint32_t* p, const uint32_t (&w)[kVecs]) {
  static_assert(kVecs == 1 || kVecs == 2 || kVecs == 4, "code words per lane");
  if constexpr (kVecs == 1) {
    store4(p, w[0]);
  } else if constexpr (kVecs == 2) {
    const v2u v = {w[0], w[1]};
    __builtin_nontemporal_store(v, (HKV_GLOBAL v2u*)p);
  } else {
    const v4u v = {w[0], w[1], w[2], w[3]};
    store16((HKV_GLOBAL v4u*)p, v);
  }
}

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// One decoded value: the low code byte times the row scale, with a NaN
// (possible only for an object the encoder did not write) written as the
// default quiet NaN so the bytes do not depend on NaN payload propagation.
__device__ __forceinline__ uint32_t decode_bits(uint32_t code, float scale) {
  const float y = (float)(int8_t)(code & 0xFFu) * scale;
  return y != y ? 0x7FC00000u : as_uint(y);
}

// Largest value of `m` over the kLanes lanes (4, 8 or 16, aligned) that hold
// one row, in every one of them: DPP lane swaps inside quads (xor 1, xor 2),
// then the mirror inside each group of 8 (lane i with 7 - i pairs its two
// quads) and inside each row of 16 (lane i with 15 - i pairs its two
// groups of 8).  A row's lanes are active or idle together, so no read
// crosses into a lane of another row.
template <uint32_t kLanes>
__device__ __forceinline__ float row_max(float m) {
  static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16, "lanes per row");
  m = fmaxf(m, as_float(__builtin_amdgcn_update_dpp(0, (int)as_uint(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, as_float(__builtin_amdgcn_update_dpp(0, (int)as_uint(m), 0x4E, 0xF, 0xF, false)));
  if (kLanes >= 8)
    m = fmaxf(m, as_float(__builtin_amdgcn_update_dpp(0, (int)as_uint(m), 0x141, 0xF, 0xF, false)));
  if (kLanes >= 16)
    m = fmaxf(m, as_float(__builtin_amdgcn_update_dpp(0, (int)as_uint(m), 0x140, 0xF, 0xF, false)));
  return m;
}

// INT8 codec of one item's recurrent-state rows (a KDA page under the
// codec: conv part, then fp32 rows of kD values).  kLanes lanes hold a row:
// lane `sub` holds the row's 16-byte vectors sub, sub + kLanes, ... (so the
// kLanes lanes of a row read 16 * kLanes contiguous bytes per load) and the
// matching 4-code words.  All of a lane's loads are issued before any use.
// Store: the row's largest finite |x| (DPP reduction), then 4 codes per
// vector; a lane computes all its code words before it stores any, so the
// stores that fill one 128-byte line of codes leave back to back (a
// nontemporal half-line followed much later by its other half makes the
// line leave L2 in extra pieces: 2-5% more bytes written).  Lane 0 of the
// row writes the row's scale with an ordinary store, so that the 4-byte
// scales of neighbouring items merge in L2 into whole lines.  When the
// objects are in host memory (kLine: the *_line gathers) the row's lanes
// first exchange code words, and each lane writes its run of adjacent words with
// one store: on the host link a row's codes then travel as one request
// instead of kVecs partial ones.
// Retrieve: q * s back.
// Quantisation (both sides of the parity tests take it in fp32, IEEE
// division and round-half-even): s = max|x| / 127; q = rint(x / s) clamped
// to [-127, 127]; 0 for non-finite x or s == 0 (Mooncake K3 blog, Compressed
// Checkpoint Storage: per-channel INT8 of inactive recurrent states).
template <uint32_t kD, bool kStore, bool kLine>
__device__ __forceinline__ void codec_rows(const hkv::CopyArgs& a,
                                           const HKV_CONST hkv::DevLayer* L, int32_t id,
                                           uint8_t* obj_page, uint32_t group) {
  constexpr uint32_t kLanes = hkv::codec_lanes_per_row(kD);
  constexpr uint32_t kVecs = kD / (4 * kLanes);  // 16-byte vectors per lane
  static_assert(kVecs >= 1 && kVecs * 4 * kLanes == kD, "a row splits into whole vectors");
  constexpr uint32_t kRowsPerPass = kThreads / kLanes;
  const uint32_t rows = L->codec_rows;
  const uint32_t sub = threadIdx.x & (kLanes - 1);
  const uint32_t r0 = group * a.codec_rows_per_item;
  const uint32_t r_end = r0 + a.codec_rows_per_item < rows ? r0 + a.codec_rows_per_item : rows;
  uint8_t* codes = obj_page + L->copy_bytes;
  uint8_t* scales = codes + (uint64_t)rows * kD;
  if (id < 0) {  // a null page: zeros in the object, nothing in the pool
    if (kStore) {
      zero_span(codes + (uint64_t)r0 * kD, (r_end - r0) * kD);
      zero_span(scales + (uint64_t)r0 * 4, (r_end - r0) * 4);
    }
    return;
  }
  uint8_t* recurrent = a.pool + L->pool_offset + (uint64_t)id * L->stride + L->copy_bytes;
  for (uint32_t r = r0 + threadIdx.x / kLanes; r < r_end; r += kRowsPerPass) {
    HKV_GLOBAL v4u* xp = (HKV_GLOBAL v4u*)(recurrent + (uint64_t)r * kD * 4);
    HKV_GLOBAL uint32_t* qp = (HKV_GLOBAL uint32_t*)(codes + (uint64_t)r * kD);
    HKV_GLOBAL uint32_t* sp = (HKV_GLOBAL uint32_t*)scales + r;
    if (kStore) {
      v4u raw[kVecs];
#pragma unroll
      for (uint32_t v = 0; v < kVecs; ++v)
        raw[v] = load16(xp + hkv::codec_input_vector(sub, v, kLanes));
      float m = 0.0f;
#pragma unroll
      for (uint32_t v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = as_float(raw[v][i]);
          m = fmaxf(m, __builtin_isfinite(x) ? fabsf(x) : 0.0f);
        }
      m = row_max<kLanes>(m);
      const float scale = m / 127.0f;
      uint32_t packed[kVecs];
#pragma unroll
      for (uint32_t v = 0; v < kVecs; ++v) {
        packed[v] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = as_float(raw[v][i]);
          const float t = fminf(fmaxf(rintf(x / scale), -127.0f), 127.0f);
          const int q = (scale != 0.0f && __builtin_isfinite(x)) ? (int)t : 0;
          packed[v] |= ((uint32_t)q & 0xFFu) << (8 * i);
        }
      }
      if constexpr (kLine) {
        // Objects in host memory: the host link carries a row's codes best
        // as one contiguous run, so the row's lanes swap words first (LDS
        // permutes inside the wave; a row's lanes are one aligned group).
        const uint32_t base = (threadIdx.x & 63u) - sub;
        const uint32_t slot = hkv::codec_word_vector(hkv::codec_line_word(sub, 0, kVecs), kLanes);
        uint32_t line[kVecs];
#pragma unroll
        for (uint32_t i = 0; i < kVecs; ++i) {
          const uint32_t w = hkv::codec_line_word(sub, i, kVecs);
          const int src = (int)((base + hkv::codec_word_lane(w, kLanes)) * 4u);
          uint32_t x = 0;
#pragma unroll
          for (uint32_t v = 0; v < kVecs; ++v) {
            const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)packed[v]);
            x = v == slot ? y : x;
          }
          line[i] = x;
        }
        store_words<kVecs>(qp + hkv::codec_line_word(sub, 0, kVecs), line);
      } else {
#pragma unroll
        for (uint32_t v = 0; v < kVecs; ++v)
          store4(qp + hkv::codec_input_vector(sub, v, kLanes), packed[v]);
      }
      if (sub == 0) *sp = as_uint(scale);
    } else {
      uint32_t packed[kVecs];
#pragma unroll
      for (uint32_t v = 0; v < kVecs; ++v)
        packed[v] = load4(qp + hkv::codec_input_vector(sub, v, kLanes));
      const float scale = as_float(load4(sp));
#pragma unroll
      for (uint32_t v = 0; v < kVecs; ++v) {
        v4u out;
        out.x = decode_bits(packed[v], scale);
        out.y = decode_bits(packed[v] >> 8, scale);
        out.z = decode_bits(packed[v] >> 16, scale);
        out.w = decode_bits(packed[v] >> 24, scale);
        store16(xp + hkv::codec_input_vector(sub, v, kLanes), out);
      }
    }
  }
}

// The work items of a call.  kD: 0 for a layout without the codec; else the
// KDA head_dim of an INT8 layout (16..256, powers of two), whose kind-1 items
// quantise or dequantise rows of kD values.  One kernel per head_dim keeps
// each kernel's registers to what its own codec path needs (more waves in
// flight than a kernel holding every head_dim).
template <bool kStore, uint32_t kUnroll, uint32_t kRun, uint32_t kD, bool kLine = false>
__device__ __forceinline__ void copy_items(const hkv::CopyArgs& a, const hkv::InlineTables& t) {
  const HKV_CONST hkv::DevLayer* layers = (const HKV_CONST hkv::DevLayer*)a.layers;
  const HKV_CONST uint64_t* items = (const HKV_CONST uint64_t*)a.items;
  // Per-call tables: in the workspace, or in the kernel arguments (which are
  // read through the constant address space like the workspace tables).
  const HKV_CONST int32_t* ids =
      (const HKV_CONST int32_t*)(a.ids ? a.ids
                                       : reinterpret_cast<const int32_t*>(t.words + a.inline_ids));
  const HKV_CONST uint64_t* objs =
      (const HKV_CONST uint64_t*)(a.objs ? a.objs : t.words + a.inline_objs);
  // (Selected without a null branch: a null alternative makes the compiler
  // copy the whole argument block to scratch.)  Read only if a.has_tokens.
  const HKV_CONST int32_t* tokens = (const HKV_CONST int32_t*)(
      a.chunk_tokens ? a.chunk_tokens : reinterpret_cast<const int32_t*>(t.words + a.inline_tokens));
  const uint32_t total = (uint32_t)a.total_items;
  const uint32_t first = hkv::xcd_first_item(blockIdx.x, gridDim.x, kRun, kXcds);
  for (uint32_t item = first; item < total; item += gridDim.x) {
    const uint32_t c = item / a.items_per_chunk;
    const uint64_t w = items[item - c * a.items_per_chunk];
    const uint32_t j = hkv::item_block(w);
    const HKV_CONST hkv::DevLayer* L = layers + hkv::item_layer(w);
    const int32_t id = ids[((uint64_t)c * a.n_kv_groups + L->kv_group) * a.blocks_per_chunk + j];
    uint8_t* obj = reinterpret_cast<uint8_t*>(objs[(uint64_t)c * a.n_obj_groups + L->obj_group]);
    uint8_t* obj_page = obj + L->obj_offset + (uint64_t)j * L->obj_page;
    if (hkv::item_kind(w)) {  // a codec row group of a KDA page (INT8 layouts only)
      if constexpr (kD != 0) codec_rows<kD, kStore, kLine>(a, L, id, obj_page, hkv::item_index(w));
      continue;
    }
    // the page (or the conv part under the codec): this tile's bytes, and
    // those of them that hold data
    const uint64_t span = L->copy_bytes;
    const hkv::TileSpan ts = hkv::tile_span(
        span, hkv::item_index(w), a.tile_bytes,
        hkv::live_span_bytes(id, span, L->row_bytes, a.has_tokens != 0,
                             a.has_tokens ? (int64_t)tokens[c] : 0, j, a.block_tokens));
    const uint32_t bytes = ts.bytes, live = ts.live;
    uint8_t* obj_tile = obj_page + ts.off;
    if (live) {
      uint8_t* page = a.pool + L->pool_offset + (uint64_t)id * L->stride + ts.off;
      if (kStore)
        copy_span<kUnroll>(obj_tile, page, live);
      else
        copy_span<kUnroll>(page, obj_tile, live);
    }
    if (kStore && live < bytes) zero_span(obj_tile + live, bytes - live);
  }
}

}  // namespace

// The gather (store) and scatter (retrieve) kernels: one pair for layouts
// without the codec, and one pair per head_dim for INT8 layouts, whose
// gather also comes in a line-code form for objects in host memory (a
// separate kernel, so that the form for device memory keeps its registers).
#define HKV_KERNEL_PAIR(suffix, kD)                                            \
  extern "C" __global__ __launch_bounds__(kThreads) void                       \
      hkv_store_gather##suffix(hkv::CopyArgs a, hkv::InlineTables t) {         \
    copy_items<true, kStoreUnroll, kStoreXcdRun, kD>(a, t);                    \
  }                                                                            \
  extern "C" __global__ __launch_bounds__(kThreads) void                       \
      hkv_retrieve_scatter##suffix(hkv::CopyArgs a, hkv::InlineTables t) {     \
    copy_items<false, kRetrieveUnroll, kRetrieveXcdRun, kD>(a, t);             \
  }
#define HKV_LINE_GATHER(suffix, kD)                                            \
  extern "C" __global__ __launch_bounds__(kThreads) void                       \
      hkv_store_gather##suffix##_line(hkv::CopyArgs a, hkv::InlineTables t) {  \
    copy_items<true, kStoreUnroll, kStoreXcdRun, kD, true>(a, t);              \
  }

HKV_KERNEL_PAIR(, 0)
HKV_KERNEL_PAIR(_int8_d16, 16)
HKV_KERNEL_PAIR(_int8_d32, 32)
HKV_KERNEL_PAIR(_int8_d64, 64)
HKV_KERNEL_PAIR(_int8_d128, 128)
HKV_KERNEL_PAIR(_int8_d256, 256)
HKV_LINE_GATHER(_int8_d16, 16)
HKV_LINE_GATHER(_int8_d32, 32)
HKV_LINE_GATHER(_int8_d64, 64)
HKV_LINE_GATHER(_int8_d128, 128)
HKV_LINE_GATHER(_int8_d256, 256)
#undef HKV_KERNEL_PAIR
#undef HKV_LINE_GATHER

namespace hkv {

int static_scratch(int dev, uint8_t** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    // Each device holds its own copy of the array at its own address.
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = static_cast<uint8_t*>(p);
  }
  *ptr = addr[dev];
  return 0;
}

int launch_copy(bool store, const CopyArgs& a, const InlineTables& t, uint32_t grid,
                void* stream) {
  if (grid == 0) return 0;
  struct Kernels {
    uint32_t head_dim;
    const void* store;
    const void* retrieve;
    const void* store_line;  // INT8 layouts: line-code gather (objects in host memory)
  };
#define HKV_FN(f) reinterpret_cast<const void*>(&f)
  static const Kernels kKernels[] = {
      {0, HKV_FN(hkv_store_gather), HKV_FN(hkv_retrieve_scatter), nullptr},
      {16, HKV_FN(hkv_store_gather_int8_d16), HKV_FN(hkv_retrieve_scatter_int8_d16),
       HKV_FN(hkv_store_gather_int8_d16_line)},
      {32, HKV_FN(hkv_store_gather_int8_d32), HKV_FN(hkv_retrieve_scatter_int8_d32),
       HKV_FN(hkv_store_gather_int8_d32_line)},
      {64, HKV_FN(hkv_store_gather_int8_d64), HKV_FN(hkv_retrieve_scatter_int8_d64),
       HKV_FN(hkv_store_gather_int8_d64_line)},
      {128, HKV_FN(hkv_store_gather_int8_d128), HKV_FN(hkv_retrieve_scatter_int8_d128),
       HKV_FN(hkv_store_gather_int8_d128_line)},
      {256, HKV_FN(hkv_store_gather_int8_d256), HKV_FN(hkv_retrieve_scatter_int8_d256),
       HKV_FN(hkv_store_gather_int8_d256_line)},
  };
#undef HKV_FN
  const void* fn = nullptr;
  for (const Kernels& k : kKernels)
    if (k.head_dim == a.codec_head_dim)
      fn = !store ? k.retrieve : (a.codec_line_codes && k.store_line) ? k.store_line : k.store;
  if (!fn) return (int)hipErrorInvalidValue;  // the planner admits no other head_dim
  CopyArgs arg = a;
  void* params[] = {&arg, const_cast<InlineTables*>(&t)};
  // The plain kernels need few registers and would run 8 waves per SIMD; they
  // measured best with fewer.  Reserving LDS they do not use caps a CU at 12
  // gather workgroups (160 KiB / 13 KiB) or 13 scatter workgroups (12 KiB).
  const uint32_t lds = a.codec_head_dim != 0 ? 0u : store ? kGatherLds : kScatterLds;
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(kThreads), params, lds,
                              reinterpret_cast<hipStream_t>(stream));
}

}  // namespace hkv
