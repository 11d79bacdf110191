// The library's host side through its C ABI, with no GPU: layout planning,
// layout and layer queries, workspace sizes, fingerprints and chunk keys on
// the five workloads' shapes and on many small random layouts, and every
// argument check of hkv_store_chunks, hkv_retrieve_chunks and
// hkv_move_chunks_noalloc on calls of up to 2000 chunks with fake device
// addresses.  Every check returns before any HIP call; the two kernel-side
// functions the host code links against are stubs that fail the program if
// a call ever gets that far.  Built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer by the tests.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hkv.h"
#include "hkv_launch.hpp"

static int g_reached = 0;
namespace hkv {
int launch_copy(bool, const CopyArgs&, const InlineTables&, uint32_t, void*) {
  g_reached = 1;
  return 100;  // hipErrorNoDevice
}
int static_scratch(int, uint8_t**) {
  g_reached = 1;
  return 100;
}
}  // namespace hkv

static int g_fail = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      printf(__VA_ARGS__);                       \
      printf(" [%s]\n", hkv_last_error());       \
      g_fail = 1;                                \
    }                                            \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t rnd() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}

struct Model {
  std::vector<uint8_t> is_mla;
  hkv_layout_desc d{};
};

static Model model(std::vector<uint8_t> is_mla, int heads, int hd, int conv, int mlab, int path,
                   uint64_t pool, int64_t N = 0, int64_t cmin = 1, int codec = 0) {
  Model m;
  m.is_mla = std::move(is_mla);
  hkv_layout_desc& d = m.d;
  d.model.n_layers = (int32_t)m.is_mla.size();
  d.model.kda_heads = heads;
  d.model.kda_head_dim = hd;
  d.model.kda_state_bytes = 4;
  d.model.conv_dim = conv;
  d.model.conv_kernel = 4;
  d.model.conv_bytes = 2;
  d.model.mla_width = 576;
  d.model.mla_bytes = mlab;
  d.block_size = N;
  d.chunk_min_tokens = cmin;
  d.path = path;
  d.separate_object_groups = 1;
  d.pool_bytes = pool;
  d.kda_codec = codec;
  return m;
}

static std::vector<uint8_t> kkkm(int n, int tail_mla) {
  std::vector<uint8_t> v;
  for (int i = 0; i < n; i++) v.push_back(i % 4 == 3);
  for (int i = 0; i < tail_mla; i++) v.push_back(1);
  return v;
}

// Every query, then the argument checks of the three copy entry points.
static void exercise(Model& m, int n_chunks) {
  m.d.model.is_mla = m.is_mla.data();
  hkv_layout* lay = nullptr;
  hkv_status st = hkv_layout_init(&m.d, &lay);
  if (st != HKV_OK) return;  // an invalid random layout: the error path is the check
  hkv_layout_info info{};
  CHECK(hkv_layout_info_get(lay, &info) == HKV_OK, "info");
  for (int32_t l = 0; l < info.n_layers; l++) {
    hkv_layer_info li{};
    CHECK(hkv_layer_info_get(lay, l, &li) == HKV_OK, "layer %d", l);
    CHECK(li.pool_offset + li.page_bytes <= info.pool_bytes_used, "page past pool");
  }
  hkv_layer_info li{};
  CHECK(hkv_layer_info_get(lay, info.n_layers, &li) == HKV_E_ARG, "layer past end");
  size_t ws = 0;
  CHECK(hkv_workspace_size(lay, n_chunks, &ws) == HKV_OK, "workspace");
  uint64_t fp = 0;
  CHECK(hkv_layout_fingerprint(lay, &fp) == HKV_OK, "fingerprint");
  std::vector<int32_t> toks(3 * info.chunk_tokens + 5);
  for (auto& t : toks) t = (int32_t)(rnd() % 200000);
  std::vector<uint64_t> prefix(toks.size()), keys(8);
  int64_t nc = 0;
  CHECK(hkv_chunk_keys(lay, toks.data(), (int64_t)toks.size(), 0, 1, 2, prefix.data(),
                       keys.data(), 4, &nc) == HKV_OK, "chunk keys");

  const uint64_t G = info.n_kv_groups, k = info.blocks_per_chunk, O = info.n_obj_groups;
  const uint64_t n = (uint64_t)n_chunks;
  std::vector<int32_t> ids(n * G * k);
  for (uint64_t i = 0; i < ids.size(); i++) ids[i] = (int32_t)(i % (uint64_t)info.num_blocks);
  const uintptr_t pool = uintptr_t(1) << 44;
  const uintptr_t ws_base = pool + (uintptr_t(1) << 43);
  std::vector<void*> objs(n * O);
  uintptr_t at = pool + (uintptr_t(1) << 42);
  for (uint64_t i = 0; i < n * O; i++) {
    objs[i] = reinterpret_cast<void*>(at);
    at += (info.obj_bytes[i % O] + 255) / 256 * 256 + 256;
  }
  std::vector<int32_t> ctoks(n, (int32_t)info.chunk_tokens);
  hkv_chunk_batch b{};
  b.n_chunks = n_chunks;
  b.block_ids = ids.data();
  b.objects = objs.data();
  void* P = reinterpret_cast<void*>(pool);
  void* W = reinterpret_cast<void*>(ws_base);
  const bool fits_one_launch = (G * k * 4 + 7) / 8 + O <= hkv::kInlineWords;
  // each call must fail on its planted defect, before any HIP call
  for (int store = 0; store < 2; store++) {
    auto call = [&](void* pool_ptr, void* ws_ptr, size_t ws_n) {
      return store ? hkv_store_chunks(lay, pool_ptr, &b, ws_ptr, ws_n, nullptr)
                   : hkv_retrieve_chunks(lay, pool_ptr, &b, ws_ptr, ws_n, nullptr);
    };
    CHECK(call(P, W, ws - 1) == HKV_E_WORKSPACE, "short workspace");
    CHECK(call(reinterpret_cast<void*>(pool + 8), W, ws) == HKV_E_ALIGN, "pool align");
    if (n > 1) {
      ids[n * G * k - 1] = (int32_t)info.num_blocks;
      CHECK(call(P, W, ws) == HKV_E_RANGE, "range");
      ids[n * G * k - 1] = -2;
      CHECK(call(P, W, ws) == HKV_E_RANGE, "range -2");
      ids[n * G * k - 1] = 0;
    }
    b.chunk_tokens = ctoks.data();
    ctoks[n - 1] = (int32_t)info.chunk_tokens + 1;
    CHECK(call(P, W, ws) == HKV_E_ARG, "tokens");
    ctoks[n - 1] = (int32_t)info.chunk_tokens;
    b.chunk_tokens = nullptr;
    void* keep = objs[n * O - 1];
    objs[n * O - 1] = objs[0];
    CHECK(call(P, W, ws) == HKV_E_ALIAS, "objects overlap");
    objs[n * O - 1] = reinterpret_cast<void*>(pool + 16);
    CHECK(call(P, W, ws) == HKV_E_ALIAS, "object in the pool");
    objs[n * O - 1] = keep;
    CHECK(call(P, reinterpret_cast<void*>(pool), ws) == HKV_E_ALIAS, "workspace in the pool");
    // the no-allocation entry point: the same checks, no workspace; a chunk
    // whose ids and object addresses alone exceed one launch's 3 KiB of
    // kernel arguments is refused first
    const int32_t op = store ? HKV_OP_STORE : HKV_OP_RETRIEVE;
    const hkv_status big = fits_one_launch ? HKV_OK : HKV_E_ARG;
    CHECK(hkv_move_chunks_noalloc(lay, op, reinterpret_cast<void*>(pool + 8), &b, nullptr) ==
              (big ? big : HKV_E_ALIGN), "noalloc align");
    objs[n * O - 1] = objs[0];
    CHECK(hkv_move_chunks_noalloc(lay, op, P, &b, nullptr) == (big ? big : HKV_E_ALIAS),
          "noalloc overlap");
    objs[n * O - 1] = keep;
  }
  if (n * G * k > 1 && info.num_blocks > 1) {
    // a retrieve may not name a block twice
    ids[0] = ids[n * G * k - 1] = (int32_t)(info.num_blocks - 1);
    CHECK(hkv_retrieve_chunks(lay, P, &b, W, ws, nullptr) == HKV_E_ALIAS, "duplicate id");
    CHECK(hkv_move_chunks_noalloc(lay, HKV_OP_RETRIEVE, P, &b, nullptr) ==
              (fits_one_launch ? HKV_E_ALIAS : HKV_E_ARG), "noalloc duplicate id");
  }
  CHECK(hkv_move_chunks_noalloc(lay, 7, P, &b, nullptr) == HKV_E_ARG, "bad op");
  hkv_layout_destroy(lay);
}

int main() {
  // the block-size rule on the pages' two Kimi-Linear shards
  Model tp2 = model(kkkm(24, 0), 16, 128, 6144, 2, 0, 16ull << 30);
  tp2.is_mla.push_back(0), tp2.is_mla.push_back(0), tp2.is_mla.push_back(1);
  tp2.d.model.n_layers = 27;
  tp2.d.model.is_mla = tp2.is_mla.data();
  int64_t N = 0;
  CHECK(hkv_unified_block_size(&tp2.d.model, 16, &N) == HKV_OK && N == 944, "N=944");
  Model tp1 = tp2;
  tp1.d.model.is_mla = tp1.is_mla.data();
  tp1.d.model.kda_heads = 32, tp1.d.model.conv_dim = 12288, tp1.d.path = 1;
  tp1.d.pool_bytes = 64ull << 30;
  CHECK(hkv_unified_block_size(&tp1.d.model, 16, &N) == HKV_OK && N == 1888, "N=1888");
  exercise(tp2, 512);
  exercise(tp1, 1024);
  Model k3 = model(kkkm(92, 1), 6, 128, 2304, 1, 0, 24ull << 30, 768, 1500);
  exercise(k3, 300);
  Model codec = tp1;
  codec.d.kda_codec = 1;
  exercise(codec, 2000);
  Model tiny = model({0, 0, 0, 1}, 2, 16, 96, 2, 0, 64ull * 16 * 576 * 2);
  exercise(tiny, 16);
  // random small layouts, valid or not
  for (int t = 0; t < 400; t++) {
    std::vector<uint8_t> is_mla(1 + rnd() % 12);
    for (auto& x : is_mla) x = rnd() % 3 == 0;
    const int hd = 16 << (rnd() % 5);
    Model m = model(is_mla, 1 + (int)(rnd() % 4), hd, (int)(8 * (rnd() % 64)),
                    1 + (int)(rnd() % 2), (int)(rnd() % 2), (1 + rnd() % 64) << 22, 0,
                    1 + (int64_t)(rnd() % 5000), (int)(rnd() % 2));
    m.d.tile_bytes = 4096 << (rnd() % 3);
    exercise(m, 1 + (int)(rnd() % 300));
  }
  // malformed arguments
  hkv_layout* lay = nullptr;
  CHECK(hkv_layout_init(nullptr, &lay) == HKV_E_ARG, "null desc");
  Model bad = model({0, 1}, 0, 16, 8, 2, 0, 1 << 26);
  bad.d.model.is_mla = bad.is_mla.data();
  CHECK(hkv_layout_init(&bad.d, &lay) == HKV_E_ARG, "zero heads");
  CHECK(!g_reached, "a call reached the kernels");
  printf(g_fail ? "api checks FAILED\n" : "api checks ok\n");
  return g_fail;
}
