// C ABI of the chunk store/retrieve library (declared in include/hkv.h).
//
// Per call: validate everything on the host, then launch one gather or
// scatter kernel on the caller's stream.  The call's own tables (block ids,
// object addresses, token counts) go in the kernel arguments when they fit;
// otherwise they are written into a pinned staging slot and copied into the
// caller's workspace on the same stream first.  No call synchronises the
// stream; a staging slot is reused only after the event recorded behind its
// copy has completed.
//
// hkv_move_chunks_noalloc runs the same kernels without any allocation: the
// layout's tables go into a static device array (hkv_copy.hip), which holds
// several layouts' tables at once, and the call's tables into kernel
// arguments, several launches if need be.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "hkv.h"
#include "hkv_device_tables.hpp"
#include "hkv_groups.hpp"
#include "hkv_launch.hpp"
#include "hkv_plan.hpp"
#include "hkv_scratch.hpp"

struct hkv_layout {
  hkv::Plan plan;
  // The plan's constant tables as the kernels read them: layer placements
  // (padded to 256 bytes), then the per-chunk work items.
  std::vector<uint8_t> table_image;
  // Never reused by another layout of the process: names the tables that the
  // static scratch of hkv_move_chunks_noalloc holds.
  uint64_t serial = 0;
  // The constant tables in the memory of each device the layout has been
  // used on, uploaded by the first call there and freed with the layout.
  mutable std::mutex mu;
  mutable std::map<int, void*> dev_tables;
  ~hkv_layout();
};

namespace {

thread_local std::string t_last_error;

hkv_status set_error(hkv_status st, const std::string& msg) {
  t_last_error = msg;
  return st;
}

hkv_status hip_error(hipError_t e, const char* what) {
  return set_error(HKV_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                  hipGetErrorString(e) + ")");
}

// HKV_TRACE=1 in the environment: one line on stderr per layout and per
// call (the layout's N, chunk size and placements; a call's chunks, launches,
// work items and bytes), like the engine's own log line naming the block size
// it settled on.
bool trace_on() {
  static const bool on = [] {
    const char* v = std::getenv("HKV_TRACE");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

// ---------------------------------------------------------------- staging
// A few pinned host buffers per device, used round-robin.  Each remembers
// the event recorded after the copy that reads it, and has its own lock: a
// call that must wait for its slot's earlier copy holds only that slot.
constexpr unsigned kSlots = 8;

struct Slot {
  std::mutex mu;
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

struct Ring {
  std::atomic<unsigned> next{0};
  Slot slot[kSlots];
};

std::mutex g_rings_mu;
std::map<int, std::unique_ptr<Ring>>* g_rings = new std::map<int, std::unique_ptr<Ring>>();

Ring* ring_for(int dev) {
  std::lock_guard<std::mutex> g(g_rings_mu);
  auto& r = (*g_rings)[dev];
  if (!r) r.reset(new Ring());
  return r.get();
}

// Makes `dev` current for the scope, restoring the previous device after.
struct DeviceScope {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceScope(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceScope() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// The device a call's work goes to: the stream's, or the current one for
// the default stream.
hkv_status stream_device(hipStream_t stream, int* dev) {
  const hipError_t e = stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
  return e == hipSuccess ? HKV_OK : hip_error(e, "finding the stream's device");
}

// Copies `bytes` bytes of `fill`-written staging into `dst` on `stream`
// (whose device is `dev`).
template <class Fill>
hkv_status upload(int dev, void* dst, size_t bytes, hipStream_t stream, Fill fill) {
  hipError_t e = hipSuccess;
  DeviceScope scope(dev);
  if (scope.err != hipSuccess) return hip_error(scope.err, "selecting the stream's device");
  Ring* ring = ring_for(dev);
  Slot& s = ring->slot[ring->next.fetch_add(1, std::memory_order_relaxed) % kSlots];
  std::lock_guard<std::mutex> g(s.mu);
  if (s.pending) {
    e = hipEventSynchronize(s.done);
    if (e != hipSuccess) return hip_error(e, "waiting for a staging slot");
    s.pending = false;
  }
  if (s.cap < bytes) {
    if (s.host) {
      e = hipHostFree(s.host);
      s.host = nullptr;
      s.cap = 0;
      if (e != hipSuccess) return hip_error(e, "hipHostFree (staging)");
    }
    const size_t cap = std::max<size_t>(bytes, size_t(64) << 10);
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_error(e, "hipHostMalloc (staging)");
    s.cap = cap;
  }
  if (!s.done) {
    e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_error(e, "hipEventCreate (staging)");
  }
  fill(static_cast<uint8_t*>(s.host));
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_error(e, "hipMemcpyAsync (tables)");
  e = hipEventRecord(s.done, stream);
  if (e != hipSuccess) {
    // Without the event the slot's copy cannot be tracked: let it finish
    // before the slot can be filled again.
    (void)hipStreamSynchronize(stream);
    return hip_error(e, "hipEventRecord (staging)");
  }
  s.pending = true;
  return HKV_OK;
}

// ---------------------------------------------------------------- validation
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;
  const char* what;
};

// Per-thread buffers of the checks, kept from call to call so that a call no
// larger than the thread's earlier ones allocates nothing on the host either.
struct CheckBuffers {
  std::vector<int32_t> ids;
  std::vector<Span> spans;
};
thread_local CheckBuffers t_check;

hkv_status check_disjoint(std::vector<Span>& spans) {
  std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].lo < spans[i - 1].hi)
      return set_error(HKV_E_ALIAS, std::string(spans[i - 1].what) + " overlaps " +
                                        spans[i].what);
  return HKV_OK;
}

// The batch's pointers, counts and the engine.  Sets *done for an empty batch.
hkv_status check_batch_shape(bool store, const hkv_layout* layout, const void* pool,
                             const hkv_chunk_batch* b, bool* done) {
  *done = false;
  if (!layout || !b) return set_error(HKV_E_ARG, "layout and batch must not be NULL");
  if (b->n_chunks < 0) return set_error(HKV_E_ARG, "n_chunks must be >= 0");
  if (b->n_chunks == 0) {
    *done = true;
    return HKV_OK;
  }
  if (!pool || !b->block_ids || !b->objects)
    return set_error(HKV_E_ARG, "pool, block_ids and objects must not be NULL");
  const hkv::Plan& p = layout->plan;
  if (b->engine != HKV_ENGINE_KERNEL && b->engine != HKV_ENGINE_DMA)
    return set_error(HKV_E_ARG, "engine must be HKV_ENGINE_KERNEL or HKV_ENGINE_DMA");
  if (b->engine == HKV_ENGINE_DMA && store)
    return set_error(HKV_E_ARG, "the DMA engine serves retrieves only (a store zero-fills "
                                "object bytes)");
  if (b->engine == HKV_ENGINE_DMA && p.kda_codec)
    return set_error(HKV_E_ARG, "the DMA engine copies bytes; an INT8 layout retrieves "
                                "through the scatter kernel, which decodes");
  if ((uint64_t)b->n_chunks * p.items.size() > 0x7FFFFFFFull)
    return set_error(HKV_E_ARG, "too many tiles in one call; split the batch");
  return HKV_OK;
}

// Object pointers, block ids, token counts, distinct retrieve targets, and
// disjoint buffers (pool, objects and, if given, the workspace span).
hkv_status check_batch_contents(bool store, const hkv::Plan& p, const void* pool,
                                const hkv_chunk_batch* b, const void* ws, uint64_t ws_need) {
  const uint64_t n = (uint64_t)b->n_chunks;
  const uint64_t G = (uint64_t)p.n_kv_groups, k = (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  for (uint64_t i = 0; i < n * O; ++i) {
    if (!b->objects[i]) return set_error(HKV_E_ARG, "object pointer is NULL");
    if (!aligned16(b->objects[i]))
      return set_error(HKV_E_ALIGN, "object pointer is not 16-byte aligned");
  }
  const int32_t* ids = b->block_ids;
  const uint64_t n_ids = n * G * k;
  for (uint64_t i = 0; i < n_ids; ++i)
    if (ids[i] != HKV_NULL_BLOCK && (ids[i] < 0 || ids[i] >= p.num_blocks))
      return set_error(HKV_E_RANGE, "block id " + std::to_string(ids[i]) + " outside [0, " +
                                        std::to_string(p.num_blocks) + ")");
  if (b->chunk_tokens)
    for (uint64_t c = 0; c < n; ++c)
      if (b->chunk_tokens[c] < 0 || b->chunk_tokens[c] > p.chunk_tokens)
        return set_error(HKV_E_ARG, "chunk_tokens[" + std::to_string(c) + "] = " +
                                        std::to_string(b->chunk_tokens[c]) + " outside [0, " +
                                        std::to_string(p.chunk_tokens) + "]");
  if (!store) {
    // One block-id space for all groups: distinct ids <=> disjoint writes.
    // Null ids write nothing.  Sorting a copy costs O(ids log ids), whatever
    // the pool's size.
    std::vector<int32_t>& v = t_check.ids;
    v.clear();
    for (uint64_t i = 0; i < n_ids; ++i)
      if (ids[i] != HKV_NULL_BLOCK) v.push_back(ids[i]);
    std::sort(v.begin(), v.end());
    for (size_t i = 1; i < v.size(); ++i)
      if (v[i] == v[i - 1])
        return set_error(HKV_E_ALIAS, "retrieve target block id " + std::to_string(v[i]) +
                                          " appears twice in one call");
  }
  std::vector<Span>& spans = t_check.spans;
  spans.clear();
  const uintptr_t pb = reinterpret_cast<uintptr_t>(pool);
  spans.push_back({pb, pb + p.pool_used, "the pool"});
  if (ws) {
    const uintptr_t wb = reinterpret_cast<uintptr_t>(ws);
    spans.push_back({wb, wb + ws_need, "the workspace"});
  }
  for (uint64_t c = 0; c < n; ++c)
    for (uint64_t o = 0; o < O; ++o) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(b->objects[c * O + o]);
      if (p.obj_bytes[o]) spans.push_back({a, a + p.obj_bytes[o], "an object"});
    }
  return check_disjoint(spans);
}

// The stream's device and whether the stream is capturing.
hkv_status stream_state(void* stream, int* dev, bool* capturing) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hkv_status st = stream_device(s, dev);
  if (st != HKV_OK) return st;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (s) {
    const hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return hip_error(e, "querying the stream's capture status");
  }
  *capturing = cap != hipStreamCaptureStatusNone;
  return HKV_OK;
}

// ---------------------------------------------------------------- layout tables
uint64_t layer_table_bytes(const hkv::Plan& p) {
  return hkv::align256(p.dev_layers.size() * sizeof(hkv::DevLayer));
}

void build_table_image(hkv_layout* lay) {
  const hkv::Plan& p = lay->plan;
  const uint64_t lb = layer_table_bytes(p), ib = p.items.size() * sizeof(uint64_t);
  lay->table_image.assign(lb + ib, 0);
  std::memcpy(lay->table_image.data(), p.dev_layers.data(),
              p.dev_layers.size() * sizeof(hkv::DevLayer));
  std::memcpy(lay->table_image.data() + lb, p.items.data(), ib);
}

// The layout's constant tables on `dev`: uploaded (synchronously) by the
// first call there, which therefore cannot be a captured one.
hkv_status layout_tables(const hkv_layout* lay, int dev, bool capturing, const uint8_t** out) {
  std::lock_guard<std::mutex> g(lay->mu);
  auto it = lay->dev_tables.find(dev);
  if (it != lay->dev_tables.end()) {
    *out = static_cast<const uint8_t*>(it->second);
    return HKV_OK;
  }
  if (capturing)
    return set_error(HKV_E_CAPTURE, "the first call of a layout on a device uploads its tables "
                                    "synchronously; make one call there before capturing");
  DeviceScope scope(dev);
  if (scope.err != hipSuccess) return hip_error(scope.err, "selecting the stream's device");
  const size_t bytes = lay->table_image.size();
  void* d = nullptr;
  hipError_t e = hipMalloc(&d, bytes);
  if (e != hipSuccess) return hip_error(e, "hipMalloc (layout tables)");
  e = hipMemcpy(d, lay->table_image.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return hip_error(e, "hipMemcpy (layout tables)");
  }
  lay->dev_tables[dev] = d;
  *out = static_cast<const uint8_t*>(d);
  return HKV_OK;
}

// ---------------------------------------------------------------- launches
// Kernel arguments for a launch over `n` chunks of `n_items` items each, with
// the layer and item tables at `layers` / `items`; the per-call table
// pointers are left null (inline) for the caller to fill.
hkv::CopyArgs base_args(const hkv::Plan& p, const void* pool, const uint8_t* layers,
                        const uint8_t* items, uint64_t n_items, uint64_t n, bool has_tokens) {
  hkv::CopyArgs a{};
  a.pool = static_cast<uint8_t*>(const_cast<void*>(pool));
  a.layers = reinterpret_cast<const hkv::DevLayer*>(layers);
  a.items = reinterpret_cast<const uint64_t*>(items);
  a.total_items = n * n_items;
  a.block_tokens = (uint64_t)p.block_size;
  a.tile_bytes = p.tile_bytes;
  a.codec_rows_per_item = p.codec_rows_per_item;
  a.codec_head_dim = p.kda_codec ? (uint32_t)p.shapes[1] : 0u;  // kda_head_dim
  a.items_per_chunk = (uint32_t)n_items;
  a.n_kv_groups = (uint32_t)p.n_kv_groups;
  a.blocks_per_chunk = (uint32_t)p.blocks_per_chunk;
  a.n_obj_groups = (uint32_t)p.n_obj_groups;
  a.has_tokens = has_tokens ? 1u : 0u;
  return a;
}

// An INT8 store whose objects are in pinned host memory writes each row's
// codes with line-wide stores (hkv_copy.hip), which the host link carries
// in fewer requests; in device memory the plain form is faster.  The first
// object pointer decides (the bytes written are the same either way).  A
// pointer the runtime cannot place leaves the plain form, and the query's
// own error is cleared, unless the thread already had one pending.
uint32_t codec_line_codes(const hkv::Plan& p, bool store, const hkv_chunk_batch* b) {
  if (!store || !p.kda_codec || b->n_chunks <= 0) return 0;
  if (hipPeekAtLastError() != hipSuccess) return 0;
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, b->objects[0]) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return attr.type == hipMemoryTypeHost ? 1u : 0u;
}

// Enqueues one launch: one workgroup per work item, unless capped by the
// caller or by the 32-bit grid size (workgroups x threads); workgroups then
// loop over items.
hkv_status launch_one(bool store, const hkv::Plan& p, const hkv::CopyArgs& a,
                      const hkv::InlineTables& t, void* stream) {
  if (a.total_items == 0) return HKV_OK;
  uint64_t grid = a.total_items;
  if (p.max_workgroups && grid > p.max_workgroups) grid = p.max_workgroups;
  const uint64_t grid_limit = 0xFFFFFFFFull / hkv::kCopyThreads;
  if (grid > grid_limit) grid = grid_limit;
  const int e = hkv::launch_copy(store, a, t, (uint32_t)grid, stream);
  if (e != 0)
    return hip_error((hipError_t)e, store ? "launching the gather kernel"
                                          : "launching the scatter kernel");
  return HKV_OK;
}

const hkv::InlineTables kNoInlineTables{};

void trace_call(const char* entry, bool store, const hkv::Plan& p, const hkv_chunk_batch* b,
                uint64_t launches, uint64_t items, const char* tables, bool line_codes = false) {
  if (!trace_on()) return;
  std::fprintf(stderr,
               "[hkv] %s %s: %d chunks, %llu launches, %llu work items (tile %llu B), "
               "%llu payload bytes, tables %s%s\n",
               entry, store ? "store" : "retrieve", b->n_chunks, (unsigned long long)launches,
               (unsigned long long)items, (unsigned long long)p.tile_bytes,
               (unsigned long long)((uint64_t)b->n_chunks * (p.obj_bytes[0] + p.obj_bytes[1])),
               tables, line_codes ? "; line-code gather (objects in host memory)" : "");
}

// The grouped retrieve (hkv_groups.hpp): one upload of every class's tables,
// then one launch per class.  Sets *done when it took the call.
hkv_status retrieve_grouped(const hkv::Plan& p, int dev, const void* pool,
                            const hkv_chunk_batch* b, void* ws, void* stream, bool* done) {
  hkv::GroupedCall g;
  *done = hkv::plan_grouped_retrieve(p, *b, &g);
  if (!*done || g.launches.empty()) return HKV_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hkv_status st = upload(dev, ws, g.ws.total, s,
                         [&](uint8_t* h) { hkv::fill_grouped_tables(p, *b, g, h); });
  if (st != HKV_OK) return st;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const bool has_tokens = b->chunk_tokens != nullptr;
  for (const hkv::GroupLaunch& L : g.launches) {
    hkv::CopyArgs a = base_args(p, pool, wsb + g.ws.layers_off, wsb + L.items_off, L.n_items,
                                L.n_chunks, has_tokens);
    a.ids = reinterpret_cast<const int32_t*>(wsb + L.ids_off);
    a.objs = reinterpret_cast<const uint64_t*>(wsb + L.objs_off);
    a.chunk_tokens = reinterpret_cast<const int32_t*>(wsb + L.tokens_off);
    st = launch_one(false, p, a, kNoInlineTables, stream);
    if (st != HKV_OK) return st;
  }
  trace_call("hkv_retrieve_chunks", false, p, b, g.launches.size(), g.launched_items,
             "staged per class");
  return HKV_OK;
}

hkv_status run_copy(bool store, const hkv_layout* layout, const void* pool,
                    const hkv_chunk_batch* b, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  hkv_status st = check_batch_shape(store, layout, pool, b, &empty);
  if (st != HKV_OK || empty) return st;
  const hkv::Plan& p = layout->plan;
  const uint64_t n = (uint64_t)b->n_chunks;
  const uint64_t G = (uint64_t)p.n_kv_groups, k = (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  const uint64_t per_chunk = p.items.size();
  const hkv::WorkspaceLayout wl =
      hkv::workspace_layout(p.dev_layers.size(), per_chunk, n, G, k, O);
  // What hkv_workspace_size(n) promises: room for the grouped retrieve too.
  const uint64_t ws_need =
      std::max(wl.total, hkv::grouped_layout(p, hkv::kMaxCallGroups * per_chunk, n).total);
  if (!ws || ws_bytes < ws_need)
    return set_error(HKV_E_WORKSPACE, "workspace needs " + std::to_string(ws_need) + " bytes");
  if (!aligned16(pool)) return set_error(HKV_E_ALIGN, "pool pointer is not 16-byte aligned");
  if (!aligned16(ws)) return set_error(HKV_E_ALIGN, "workspace is not 16-byte aligned");
  st = check_batch_contents(store, p, pool, b, ws, ws_need);
  if (st != HKV_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  bool capturing = false;
  // Under stream capture only what a graph can replay is enqueued: DMA
  // copies between the caller's buffers, or one launch whose tables are in
  // its arguments.  A copy out of a staging slot would replay whatever the
  // ring later put in that slot.
  st = stream_state(stream, &dev, &capturing);
  if (st != HKV_OK) return st;
  const int32_t* ids = b->block_ids;
  const uint64_t n_ids = n * G * k;

  if (b->engine == HKV_ENGINE_DMA) {
    // One copy per run of pages contiguous in both the object and the pool.
    std::vector<hkv::DmaRun> runs;
    hkv::plan_dma_runs(p, *b, reinterpret_cast<uintptr_t>(pool), &runs);
    DeviceScope scope(dev);
    if (scope.err != hipSuccess) return hip_error(scope.err, "selecting the stream's device");
    for (const hkv::DmaRun& r : runs) {
      const hipError_t e = hipMemcpyAsync(reinterpret_cast<void*>(r.dst),
                                          reinterpret_cast<const void*>(r.src), r.bytes,
                                          hipMemcpyDefault, s);
      if (e != hipSuccess) return hip_error(e, "hipMemcpyAsync (DMA retrieve)");
    }
    if (trace_on())
      std::fprintf(stderr, "[hkv] hkv_retrieve_chunks retrieve (DMA): %d chunks, %zu copies\n",
                   b->n_chunks, runs.size());
    return HKV_OK;
  }

  if (!store && !capturing) {
    bool any_null = false;
    for (uint64_t i = 0; i < n_ids && !any_null; ++i) any_null = ids[i] == HKV_NULL_BLOCK;
    if (any_null || b->chunk_tokens) {
      bool done = false;
      st = retrieve_grouped(p, dev, pool, b, ws, stream, &done);
      if (st != HKV_OK || done) return st;
    }
  }

  const uint8_t* tables = nullptr;
  st = layout_tables(layout, dev, capturing, &tables);
  if (st != HKV_OK) return st;
  const bool has_tokens = b->chunk_tokens != nullptr;
  hkv::CopyArgs a =
      base_args(p, pool, tables, tables + layer_table_bytes(p), per_chunk, n, has_tokens);
  a.codec_line_codes = codec_line_codes(p, store, b);
  const char* entry = store ? "hkv_store_chunks" : "hkv_retrieve_chunks";
  // Per-call tables: in the kernel arguments when they fit (no copy ahead of
  // the launch), else uploaded into the workspace.
  {
    hkv::InlineTables t;
    if (hkv::pack_inline_tables(p, *b, &t, &a)) {
      st = launch_one(store, p, a, t, stream);
      if (st == HKV_OK)
        trace_call(entry, store, p, b, 1, a.total_items, "in the arguments", a.codec_line_codes);
      return st;
    }
  }
  if (capturing)
    return set_error(HKV_E_CAPTURE, "the call's tables do not fit in the kernel arguments, "
                                    "so it cannot be captured; split the batch");
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const uint64_t lo = wl.ids_off;  // the per-call sections: ids, objects, tokens
  st = upload(dev, wsb + lo, wl.total - lo, s, [&](uint8_t* h) {
    std::memcpy(h + (wl.ids_off - lo), ids, n_ids * sizeof(int32_t));
    uint64_t* objs = reinterpret_cast<uint64_t*>(h + (wl.objs_off - lo));
    for (uint64_t i = 0; i < n * O; ++i) objs[i] = reinterpret_cast<uintptr_t>(b->objects[i]);
    if (has_tokens) std::memcpy(h + (wl.tokens_off - lo), b->chunk_tokens, n * sizeof(int32_t));
  });
  if (st != HKV_OK) return st;
  a.ids = reinterpret_cast<const int32_t*>(wsb + wl.ids_off);
  a.objs = reinterpret_cast<const uint64_t*>(wsb + wl.objs_off);
  a.chunk_tokens = reinterpret_cast<const int32_t*>(wsb + wl.tokens_off);
  st = launch_one(store, p, a, kNoInlineTables, stream);
  if (st == HKV_OK) trace_call(entry, store, p, b, 1, a.total_items, "staged", a.codec_line_codes);
  return st;
}

// ---------------------------------------------------------------- no allocation
// The directory of each device's static scratch: which layouts' tables it
// holds, and where (hkv_scratch.hpp).  The lock and the directories are never
// destroyed, so a layout destroyed late in process exit can still drop its
// entries.
constexpr int kMaxScratchDevices = 64;
std::mutex& scratch_mu() {
  static std::mutex* m = new std::mutex();
  return *m;
}
hkv::ScratchDirectory* g_scratch_dir[kMaxScratchDevices] = {};
std::atomic<uint64_t> g_next_serial{1};

// The most chunks of a call whose block ids, object addresses and token
// counts fit in one launch's kernel arguments.
uint64_t inline_chunks_per_launch(const hkv::Plan& p, bool has_tokens) {
  const uint64_t ids = (uint64_t)p.n_kv_groups * (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  auto words = [&](uint64_t m) {
    return (m * ids * sizeof(int32_t) + 7) / 8 + m * O +
           (has_tokens ? (m * sizeof(int32_t) + 7) / 8 : 0);
  };
  uint64_t m = hkv::kInlineWords;  // an upper bound: a chunk takes at least one word
  while (m > 0 && words(m) > hkv::kInlineWords) --m;
  return m;
}

hkv_status move_noalloc(bool store, const hkv_layout* layout, void* pool,
                        const hkv_chunk_batch* b, void* stream) {
  bool empty = false;
  hkv_status st = check_batch_shape(store, layout, pool, b, &empty);
  if (st != HKV_OK || empty) return st;
  if (b->engine != HKV_ENGINE_KERNEL)
    return set_error(HKV_E_ARG, "hkv_move_chunks_noalloc runs the kernels only "
                                "(engine must be HKV_ENGINE_KERNEL)");
  const hkv::Plan& p = layout->plan;
  const bool has_tokens = b->chunk_tokens != nullptr;
  const uint64_t per_launch = inline_chunks_per_launch(p, has_tokens);
  if (per_launch == 0)
    return set_error(HKV_E_ARG, "one chunk's block ids and object addresses exceed the "
                                "kernel-argument block");
  const uint64_t table_bytes = layout->table_image.size();
  if (table_bytes > hkv::kStaticScratchBytes)
    return set_error(HKV_E_WORKSPACE, "the layout's tables need " + std::to_string(table_bytes) +
                                          " bytes; the static scratch holds " +
                                          std::to_string(hkv::kStaticScratchBytes));
  if (!aligned16(pool)) return set_error(HKV_E_ALIGN, "pool pointer is not 16-byte aligned");
  st = check_batch_contents(store, p, pool, b, nullptr, 0);
  if (st != HKV_OK) return st;

  int dev = 0;
  bool capturing = false;
  st = stream_state(stream, &dev, &capturing);
  if (st != HKV_OK) return st;
  if (dev < 0 || dev >= kMaxScratchDevices)
    return set_error(HKV_E_ARG, "device index beyond the static scratch's device table");
  uint8_t* scratch = nullptr;
  {
    DeviceScope scope(dev);
    if (scope.err != hipSuccess) return hip_error(scope.err, "selecting the stream's device");
    const int e = hkv::static_scratch(dev, &scratch);
    if (e != 0) return hip_error((hipError_t)e, "hipGetSymbolAddress (static scratch)");
  }
  uint64_t table_off = 0;
  {
    // The layout's tables into the scratch, unless they are there already.
    // The source is the layout's own host image; the stream is then drained
    // so that work on any other stream sees the tables whole.
    std::lock_guard<std::mutex> g(scratch_mu());
    if (!g_scratch_dir[dev]) g_scratch_dir[dev] = new hkv::ScratchDirectory(hkv::kStaticScratchBytes);
    hkv::ScratchDirectory& dir = *g_scratch_dir[dev];
    hkv::ScratchDirectory::Entry* ent = dir.find(layout->serial);
    if (!ent) {
      if (capturing)
        return set_error(HKV_E_CAPTURE, "this layout's tables are not in the static scratch of "
                                        "the stream's device; make one call with it there "
                                        "before capturing");
      int evicted = 0;
      ent = dir.reserve(layout->serial, table_bytes, &evicted);
      if (!ent)
        return set_error(HKV_E_WORKSPACE, "no room in the static scratch: the layouts that "
                                          "captured calls use fill it (destroy one first)");
      hipStream_t s = reinterpret_cast<hipStream_t>(stream);
      DeviceScope scope(dev);
      hipError_t e = scope.err;
      if (e == hipSuccess)
        e = hipMemcpyAsync(scratch + ent->off, layout->table_image.data(), table_bytes,
                           hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) {
        dir.drop(layout->serial);
        return hip_error(e, "copying the layout's tables into the static scratch");
      }
      if (trace_on())
        std::fprintf(stderr,
                     "[hkv] static scratch of device %d: %llu bytes of tables copied in at "
                     "offset %llu, %d layout(s) evicted\n",
                     dev, (unsigned long long)table_bytes, (unsigned long long)ent->off, evicted);
    }
    dir.touch(ent, capturing);
    table_off = ent->off;
  }
  const uint64_t n = (uint64_t)b->n_chunks;
  const uint64_t Gk = (uint64_t)p.n_kv_groups * (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  const uint8_t* layers = scratch + table_off;
  const uint8_t* items = layers + layer_table_bytes(p);
  const uint32_t line_codes = codec_line_codes(p, store, b);
  uint64_t launches = 0;
  for (uint64_t c0 = 0; c0 < n; c0 += per_launch) {
    const uint64_t m = std::min(per_launch, n - c0);
    hkv_chunk_batch part{};
    part.n_chunks = (int32_t)m;
    part.block_ids = b->block_ids + c0 * Gk;
    part.objects = b->objects + c0 * O;
    part.chunk_tokens = has_tokens ? b->chunk_tokens + c0 : nullptr;
    part.engine = HKV_ENGINE_KERNEL;
    hkv::CopyArgs a = base_args(p, pool, layers, items, p.items.size(), m, has_tokens);
    a.codec_line_codes = line_codes;
    hkv::InlineTables t;
    if (!hkv::pack_inline_tables(p, part, &t, &a))
      return set_error(HKV_E_ARG, "internal: a launch's tables do not fit its arguments");
    st = launch_one(store, p, a, t, stream);
    if (st != HKV_OK) return st;
    ++launches;
  }
  trace_call("hkv_move_chunks_noalloc", store, p, b, launches, n * p.items.size(),
             "in the arguments; layout tables in the static scratch", line_codes != 0);
  return HKV_OK;
}

}  // namespace

hkv_layout::~hkv_layout() {
  for (auto& kv : dev_tables) {
    DeviceScope scope(kv.first);
    if (scope.err == hipSuccess) (void)hipFree(kv.second);
  }
  // its place in each device's static scratch is free again
  std::lock_guard<std::mutex> g(scratch_mu());
  for (hkv::ScratchDirectory* dir : g_scratch_dir)
    if (dir) dir->drop(serial);
}

extern "C" {

hkv_status hkv_unified_block_size(const hkv_model* model, int32_t align_tokens, int64_t* n_out) {
  if (!model || !n_out) return set_error(HKV_E_ARG, "model and n_out must not be NULL");
  if (align_tokens != 0 && align_tokens != 16)
    return set_error(HKV_E_ARG, "only a 16-token step is supported");
  std::string err;
  hkv_status st = hkv::unified_block_size(*model, n_out, &err);
  return st == HKV_OK ? st : set_error(st, err);
}

hkv_status hkv_layout_init(const hkv_layout_desc* desc, hkv_layout** out) {
  if (!desc || !out) return set_error(HKV_E_ARG, "desc and out must not be NULL");
  std::unique_ptr<hkv_layout> lay(new (std::nothrow) hkv_layout());
  if (!lay) return set_error(HKV_E_ARG, "out of host memory");
  std::string err;
  hkv_status st = hkv::make_plan(*desc, &lay->plan, &err);
  if (st != HKV_OK) return set_error(st, err);
  build_table_image(lay.get());
  lay->serial = g_next_serial.fetch_add(1, std::memory_order_relaxed);
  if (trace_on()) {
    const hkv::Plan& p = lay->plan;
    std::fprintf(stderr,
                 "[hkv] layout: block size N=%lld tokens, chunk C=%lld (k=%d), path %c, "
                 "%d KV groups, %d object groups, %lld blocks, stride %llu B, pool %llu B used, "
                 "chunk payload %llu B, %zu work items per chunk (tile %llu B)%s\n",
                 (long long)p.block_size, (long long)p.chunk_tokens, p.blocks_per_chunk,
                 p.path == 0 ? 'A' : 'B', p.n_kv_groups, p.n_obj_groups,
                 (long long)p.num_blocks, (unsigned long long)p.block_stride,
                 (unsigned long long)p.pool_used,
                 (unsigned long long)(p.obj_bytes[0] + p.obj_bytes[1]), p.items.size(),
                 (unsigned long long)p.tile_bytes, p.kda_codec ? ", INT8 KDA codec" : "");
  }
  *out = lay.release();
  return HKV_OK;
}

void hkv_layout_destroy(hkv_layout* layout) { delete layout; }

hkv_status hkv_layout_info_get(const hkv_layout* layout, hkv_layout_info* out) {
  if (!layout || !out) return set_error(HKV_E_ARG, "layout and out must not be NULL");
  const hkv::Plan& p = layout->plan;
  std::memset(out, 0, sizeof(*out));
  out->block_size = p.block_size;
  out->chunk_tokens = p.chunk_tokens;
  out->blocks_per_chunk = p.blocks_per_chunk;
  out->n_layers = (int32_t)p.layers.size();
  out->n_kv_groups = p.n_kv_groups;
  out->n_obj_groups = p.n_obj_groups;
  out->num_blocks = p.num_blocks;
  out->path = p.path;
  out->n_slabs = p.n_slabs;
  out->unified_page_bytes = p.unified_page;
  out->block_stride = p.block_stride;
  out->pool_bytes_used = p.pool_used;
  out->obj_bytes[0] = p.obj_bytes[0];
  out->obj_bytes[1] = p.obj_bytes[1];
  out->chunk_payload_bytes = p.obj_bytes[0] + p.obj_bytes[1];
  out->kda_codec = p.kda_codec;
  return HKV_OK;
}

hkv_status hkv_layer_info_get(const hkv_layout* layout, int32_t layer, hkv_layer_info* out) {
  if (!layout || !out) return set_error(HKV_E_ARG, "layout and out must not be NULL");
  const hkv::Plan& p = layout->plan;
  if (layer < 0 || layer >= (int32_t)p.layers.size())
    return set_error(HKV_E_ARG, "layer index out of range");
  const hkv::LayerPlacement& x = p.layers[layer];
  out->is_mla = x.is_mla;
  out->kv_group = x.kv_group;
  out->obj_group = x.obj_group;
  out->slot = x.slot;
  out->page_bytes = x.page;
  out->reserved_bytes = x.reserved;
  out->pool_offset = x.pool_offset;
  out->stride = x.stride;
  out->obj_offset = x.obj_offset;
  out->obj_page_bytes = x.obj_page;
  return HKV_OK;
}

hkv_status hkv_workspace_size(const hkv_layout* layout, int32_t max_chunks, size_t* bytes) {
  if (!layout || !bytes) return set_error(HKV_E_ARG, "layout and bytes must not be NULL");
  if (max_chunks < 0) return set_error(HKV_E_ARG, "max_chunks must be >= 0");
  const hkv::Plan& p = layout->plan;
  const uint64_t single = hkv::workspace_layout(p.dev_layers.size(), p.items.size(),
                                                (uint64_t)max_chunks, (uint64_t)p.n_kv_groups,
                                                (uint64_t)p.blocks_per_chunk,
                                                (uint64_t)p.n_obj_groups)
                              .total;
  // A retrieve with null ids or partial chunks may use up to kMaxCallGroups
  // item lists (one per class of chunks).
  const uint64_t grouped =
      hkv::grouped_layout(p, hkv::kMaxCallGroups * p.items.size(), (uint64_t)max_chunks).total;
  *bytes = (size_t)std::max(single, grouped);
  return HKV_OK;
}

hkv_status hkv_store_chunks(const hkv_layout* layout, const void* pool,
                            const hkv_chunk_batch* batch, void* workspace, size_t ws_bytes,
                            void* stream) {
  return run_copy(true, layout, pool, batch, workspace, ws_bytes, stream);
}

hkv_status hkv_retrieve_chunks(const hkv_layout* layout, void* pool,
                               const hkv_chunk_batch* batch, void* workspace, size_t ws_bytes,
                               void* stream) {
  return run_copy(false, layout, pool, batch, workspace, ws_bytes, stream);
}

hkv_status hkv_move_chunks_noalloc(const hkv_layout* layout, int32_t op, void* pool,
                                   const hkv_chunk_batch* batch, void* stream) {
  if (op != HKV_OP_STORE && op != HKV_OP_RETRIEVE)
    return set_error(HKV_E_ARG, "op must be HKV_OP_STORE or HKV_OP_RETRIEVE");
  return move_noalloc(op == HKV_OP_STORE, layout, pool, batch, stream);
}

hkv_status hkv_layout_fingerprint(const hkv_layout* layout, uint64_t* out) {
  if (!layout || !out) return set_error(HKV_E_ARG, "layout and out must not be NULL");
  *out = hkv::object_fingerprint(layout->plan);
  return HKV_OK;
}

hkv_status hkv_chunk_keys(const hkv_layout* layout, const int32_t* tokens, int64_t n_tokens,
                          int32_t hash_block_tokens, uint64_t root, uint64_t rank_tag,
                          uint64_t* prefix_hashes_out, uint64_t* keys_out, int32_t max_chunks,
                          int64_t* n_chunks_out) {
  if (!layout) return set_error(HKV_E_ARG, "layout must not be NULL");
  std::string err;
  hkv_status st = hkv::chunk_keys(layout->plan, tokens, n_tokens, hash_block_tokens, root,
                                  rank_tag, prefix_hashes_out, keys_out, max_chunks,
                                  n_chunks_out, &err);
  return st == HKV_OK ? st : set_error(st, err);
}

const char* hkv_last_error(void) { return t_last_error.c_str(); }

}  // extern "C"
