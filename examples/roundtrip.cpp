// A store and a retrieve through the C ABI alone (include/hkv.h and the HIP
// runtime; no Python, no torch): chunks of a small hybrid KDA+MLA layout are
// gathered from a pool into chunk objects, then scattered into newly drawn
// block ids of a second, zeroed pool.  Every page must come back byte for
// byte, and nothing else in the second pool may change (the store/retrieve
// round trip of the LMCache "Hybrid Attention Models" page: a retrieved
// state is the stored one).  The same round trip then runs through the
// no-allocation entry point, captured into a HIP graph and replayed.
//
// Build:  hipcc --offload-arch=gfx950 -O2 -std=c++17 -I include \
//           examples/roundtrip.cpp -L retrieve_store_chunk_amd -lhkv \
//           -Wl,-rpath,'$ORIGIN/../retrieve_store_chunk_amd' -o examples/roundtrip
// Run:    examples/roundtrip        (prints "roundtrip ok: ..." and exits 0)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "hkv.h"

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
      return 1;                                                                    \
    }                                                                              \
  } while (0)
#define HKV_OK_(x)                                                                 \
  do {                                                                             \
    hkv_status s_ = (x);                                                           \
    if (s_ != HKV_OK) {                                                            \
      std::fprintf(stderr, "%s: status %d: %s\n", #x, s_, hkv_last_error());       \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

int main() {
  // Four layers, three KDA then one MLA; per-rank KDA state 2 x 16 x 16 fp32
  // plus a (96, 3) bf16 conv state; 576 bf16 latent values per MLA token.
  const uint8_t is_mla[4] = {0, 0, 0, 1};
  hkv_layout_desc d;
  std::memset(&d, 0, sizeof d);
  d.model.n_layers = 4;
  d.model.is_mla = is_mla;
  d.model.kda_heads = 2;
  d.model.kda_head_dim = 16;
  d.model.kda_state_bytes = 4;
  d.model.conv_dim = 96;
  d.model.conv_kernel = 4;
  d.model.conv_bytes = 2;
  d.model.mla_width = 576;
  d.model.mla_bytes = 2;
  d.chunk_min_tokens = 40;  // negotiated to the next multiple of N
  d.path = 1;               // packed pool
  d.separate_object_groups = 1;
  d.pool_bytes = 64ull << 20;
  hkv_layout* lay = nullptr;
  HKV_OK_(hkv_layout_init(&d, &lay));
  hkv_layout_info info;
  HKV_OK_(hkv_layout_info_get(lay, &info));
  std::vector<hkv_layer_info> layers(info.n_layers);
  for (int l = 0; l < info.n_layers; ++l) HKV_OK_(hkv_layer_info_get(lay, l, &layers[l]));

  const int n = 24;  // chunks per call
  const int G = info.n_kv_groups, k = info.blocks_per_chunk, O = info.n_obj_groups;
  const size_t used = info.pool_bytes_used;
  if ((int64_t)2 * n * G * k > info.num_blocks) {
    std::fprintf(stderr, "pool too small\n");
    return 1;
  }

  // Seeded pool bytes; store ids and retrieve ids drawn from one shuffle, so
  // the retrieve targets are fresh ids.
  std::mt19937_64 rng(0x48B0000);
  std::vector<uint8_t> src(used);
  for (auto& b : src) b = (uint8_t)rng();
  std::vector<int32_t> perm(info.num_blocks);
  for (int64_t i = 0; i < info.num_blocks; ++i) perm[i] = (int32_t)i;
  std::shuffle(perm.begin(), perm.end(), rng);
  std::vector<int32_t> store_ids(perm.begin(), perm.begin() + n * G * k);
  std::vector<int32_t> retr_ids(perm.begin() + n * G * k, perm.begin() + 2 * n * G * k);

  uint8_t *pool_a = nullptr, *pool_b = nullptr, *objs = nullptr, *ws = nullptr;
  size_t obj_stride[2] = {0, 0}, chunk_bytes = 0;
  for (int o = 0; o < O; ++o) {
    obj_stride[o] = (info.obj_bytes[o] + 255) / 256 * 256;
    chunk_bytes += obj_stride[o];
  }
  size_t ws_bytes = 0;
  HKV_OK_(hkv_workspace_size(lay, n, &ws_bytes));
  HIP_OK(hipMalloc(&pool_a, used));
  HIP_OK(hipMalloc(&pool_b, used));
  HIP_OK(hipMalloc(&objs, chunk_bytes * n));
  HIP_OK(hipMalloc(&ws, ws_bytes < 256 ? 256 : ws_bytes));
  HIP_OK(hipMemcpy(pool_a, src.data(), used, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(pool_b, 0, used));
  std::vector<void*> obj_ptrs(n * O);
  for (int c = 0; c < n; ++c) {
    size_t off = c * chunk_bytes;
    for (int o = 0; o < O; ++o) {
      obj_ptrs[c * O + o] = objs + off;
      off += obj_stride[o];
    }
  }
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  hkv_chunk_batch b;
  std::memset(&b, 0, sizeof b);
  b.n_chunks = n;
  b.objects = obj_ptrs.data();
  b.engine = HKV_ENGINE_KERNEL;
  b.block_ids = store_ids.data();
  HKV_OK_(hkv_store_chunks(lay, pool_a, &b, ws, ws_bytes, stream));
  b.block_ids = retr_ids.data();
  HKV_OK_(hkv_retrieve_chunks(lay, pool_b, &b, ws, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));

  std::vector<uint8_t> got(used);
  HIP_OK(hipMemcpy(got.data(), pool_b, used, hipMemcpyDeviceToHost));
  // Expected second pool: zeros, plus every stored page at its retrieve id.
  std::vector<uint8_t> want(used, 0);
  size_t pages = 0;
  for (int c = 0; c < n; ++c)
    for (const hkv_layer_info& L : layers)
      for (int j = 0; j < k; ++j) {
        const size_t i = ((size_t)c * G + L.kv_group) * k + j;
        std::memcpy(want.data() + L.pool_offset + (size_t)retr_ids[i] * L.stride,
                    src.data() + L.pool_offset + (size_t)store_ids[i] * L.stride, L.page_bytes);
        ++pages;
      }
  if (std::memcmp(got.data(), want.data(), used) != 0) {
    size_t first = 0;
    while (got[first] == want[first]) ++first;
    std::fprintf(stderr, "roundtrip FAILED: first difference at pool byte %zu\n", first);
    return 1;
  }

  // The same round trip through hkv_move_chunks_noalloc (no workspace, no
  // allocation), captured once into a HIP graph and replayed: one eager call
  // first puts the layout's tables into the library's static scratch, which
  // a captured call cannot do.
  hkv_chunk_batch bs = b, br = b;
  bs.block_ids = store_ids.data();
  br.block_ids = retr_ids.data();
  HKV_OK_(hkv_move_chunks_noalloc(lay, HKV_OP_STORE, pool_a, &bs, stream));
  HIP_OK(hipStreamSynchronize(stream));
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
  const hkv_status st_s = hkv_move_chunks_noalloc(lay, HKV_OP_STORE, pool_a, &bs, stream);
  const hkv_status st_r = hkv_move_chunks_noalloc(lay, HKV_OP_RETRIEVE, pool_b, &br, stream);
  HIP_OK(hipStreamEndCapture(stream, &graph));
  HKV_OK_(st_s);
  HKV_OK_(st_r);
  HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  const int replays = 3;
  for (int rep = 0; rep < replays; ++rep) {
    // fresh destinations before each replay (cleared outside the graph)
    HIP_OK(hipMemset(pool_b, 0, used));
    HIP_OK(hipMemset(objs, 0, chunk_bytes * n));
    HIP_OK(hipGraphLaunch(exec, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(got.data(), pool_b, used, hipMemcpyDeviceToHost));
    if (std::memcmp(got.data(), want.data(), used) != 0) {
      std::fprintf(stderr, "roundtrip FAILED: graph replay %d differs\n", rep);
      return 1;
    }
  }
  // Host time to enqueue one call (validation, tables in the kernel
  // arguments, launch), and the time of one replay of the captured pair.
  const int reps = 200;
  hipEvent_t e0, e1;
  HIP_OK(hipEventCreate(&e0));
  HIP_OK(hipEventCreate(&e1));
  auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < reps; ++i) HKV_OK_(hkv_store_chunks(lay, pool_a, &bs, ws, ws_bytes, stream));
  const double enqueue_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() /
      reps;
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipEventRecord(e0, stream));
  for (int i = 0; i < reps; ++i) HIP_OK(hipGraphLaunch(exec, stream));
  HIP_OK(hipEventRecord(e1, stream));
  HIP_OK(hipEventSynchronize(e1));
  float ms = 0.0f;
  HIP_OK(hipEventElapsedTime(&ms, e0, e1));
  std::printf("roundtrip ok: %d chunks, %zu pages, N=%lld, C=%lld, %d KV groups, %d objects; "
              "no-allocation pair as a graph: %d replays match; %.1f us to enqueue a store, "
              "%.1f us per replay of store + retrieve\n",
              n, pages, (long long)info.block_size, (long long)info.chunk_tokens, G, O, replays,
              enqueue_us, 1e3 * ms / reps);
  HIP_OK(hipEventDestroy(e0));
  HIP_OK(hipEventDestroy(e1));
  HIP_OK(hipGraphExecDestroy(exec));
  HIP_OK(hipGraphDestroy(graph));
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(pool_a));
  HIP_OK(hipFree(pool_b));
  HIP_OK(hipFree(objs));
  HIP_OK(hipFree(ws));
  hkv_layout_destroy(lay);
  return 0;
}
