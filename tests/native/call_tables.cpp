// A call's tables as the kernels read them, replayed on the host:
//   - a grouped retrieve (one launch per class of chunks over the items that
//     write something) makes exactly the copies of the plain launch over
//     every item, reads its tables only inside the staged bytes, and writes
//     only live page bytes; it is declined past 8 classes and for whole,
//     null-free batches;
//   - the per-call tables packed into the kernel arguments read back as the
//     batch's ids, object addresses and token counts, and are packed exactly
//     when they fit;
//   - a DMA retrieve's runs move exactly the bytes of the plain launch's
//     copies, each copy inside one run at the same offset on both sides.
#include <cstdio>
#include <cstring>
#include <vector>
#include <map>
#include <tuple>
#include <random>
#include <algorithm>
#include "hkv_plan.hpp"
#include "hkv_groups.hpp"

static std::vector<uint8_t> kimi27() { std::vector<uint8_t> v; for (int i=0;i<24;i++) v.push_back(i%4==3); v.push_back(0); v.push_back(0); v.push_back(1); return v; }
static std::vector<uint8_t> k393() { std::vector<uint8_t> v; for (int i=0;i<92;i++) v.push_back(i%4==3); v.push_back(1); return v; }
#define FAIL(...) do { printf("%s: ", name); printf(__VA_ARGS__); printf("\n"); return 1; } while (0)

// (pool lo, bytes, chunk, obj group, obj offset, kind)
typedef std::tuple<uint64_t, uint64_t, uint32_t, uint32_t, uint64_t, int> Op;

// Copies one launch would make, reading its tables from `tab` (a staged
// buffer) at the given offsets, as the kernel does.
static int ops_of(const char* name, const hkv::Plan& p, const uint8_t* tab, uint64_t tab_bytes,
                  uint64_t items_off, uint64_t n_items, uint64_t ids_off, uint64_t objs_off,
                  uint64_t tokens_off, bool has_tokens, uint64_t n_chunks,
                  const std::map<uint64_t, std::pair<uint32_t,uint32_t>>& obj_of, std::vector<Op>* out) {
  const uint64_t G = p.n_kv_groups, k = p.blocks_per_chunk, O = p.n_obj_groups;
  auto need = [&](uint64_t off, uint64_t n) { return off + n <= tab_bytes; };
  if (!need(items_off, n_items * 8) || !need(ids_off, n_chunks * G * k * 4) || !need(objs_off, n_chunks * O * 8) ||
      (has_tokens && !need(tokens_off, n_chunks * 4))) FAIL("table past the staged bytes");
  const uint64_t* items = (const uint64_t*)(tab + items_off);
  const int32_t* ids = (const int32_t*)(tab + ids_off);
  const uint64_t* objs = (const uint64_t*)(tab + objs_off);
  const int32_t* toks = (const int32_t*)(tab + tokens_off);
  for (uint64_t item = 0; item < n_chunks * n_items; ++item) {
    const uint64_t c = item / n_items, r = item % n_items, w = items[r];
    const uint32_t l = hkv::item_layer(w), j = hkv::item_block(w), s = hkv::item_index(w);
    const uint32_t kind = hkv::item_kind(w);
    if (l >= p.dev_layers.size() || j >= k) FAIL("bad item");
    const hkv::DevLayer& L = p.dev_layers[l];
    const int32_t id = ids[(c * G + L.kv_group) * k + j];
    if (id != -1 && (id < 0 || id >= p.num_blocks)) FAIL("id %d out of range (tables misread?)", id);
    const uint64_t ob = objs[c * O + L.obj_group];
    auto it = obj_of.find(ob);
    if (it == obj_of.end()) FAIL("object address not one of the batch's");
    const uint32_t ch = it->second.first;
    if (it->second.second != L.obj_group) FAIL("object of the wrong group");
    const uint64_t obj_page = L.obj_offset + (uint64_t)j * L.obj_page;
    if (kind) {
      if (id < 0) continue;
      const uint32_t r0 = s * p.codec_rows_per_item;
      const uint32_t r_end = std::min<uint32_t>(r0 + p.codec_rows_per_item, L.codec_rows);
      const uint64_t lo = L.pool_offset + (uint64_t)id * L.stride + L.copy_bytes + (uint64_t)r0 * L.head_dim * 4;
      out->push_back(Op(lo, (uint64_t)(r_end - r0) * L.head_dim * 4, ch, L.obj_group, obj_page + L.copy_bytes + (uint64_t)r0 * L.head_dim, 1));
      continue;
    }
    // the kernels' own tile arithmetic (hkv_device_tables.hpp)
    const hkv::TileSpan ts = hkv::tile_span(
        L.copy_bytes, s, p.tile_bytes,
        hkv::live_span_bytes(id, L.copy_bytes, L.row_bytes, has_tokens,
                             has_tokens ? (int64_t)toks[c] : 0, j, (uint64_t)p.block_size));
    const uint64_t off = ts.off, live = ts.live;
    if (!live) continue;
    const uint64_t lo = L.pool_offset + (uint64_t)id * L.stride + off;
    if (lo + live > L.pool_offset + (uint64_t)id * L.stride + L.page || lo + live > p.pool_used) FAIL("pool write past the page");
    out->push_back(Op(lo, live, ch, L.obj_group, obj_page + off, 0));
  }
  return 0;
}

static int check(const char* name, std::vector<uint8_t> is_mla, int heads, int d, int conv, int mlab, int path,
                 uint64_t pool, int64_t N, int64_t cmin, int codec, int n, int n_patterns, int n_tok_values, unsigned seed,
                 bool expect_grouped) {
  hkv_layout_desc desc{}; desc.model.n_layers = is_mla.size(); desc.model.is_mla = is_mla.data();
  desc.model.kda_heads=heads; desc.model.kda_head_dim=d; desc.model.kda_state_bytes=4; desc.model.conv_dim=conv; desc.model.conv_kernel=4; desc.model.conv_bytes=2; desc.model.mla_width=576; desc.model.mla_bytes=mlab;
  desc.block_size=N; desc.chunk_min_tokens=cmin; desc.path=path; desc.separate_object_groups=1; desc.pool_bytes=pool; desc.kda_codec=codec;
  hkv::Plan p; std::string err;
  if (hkv::make_plan(desc, &p, &err) != HKV_OK) FAIL("plan: %s", err.c_str());
  const uint64_t G = p.n_kv_groups, k = p.blocks_per_chunk, O = p.n_obj_groups;
  std::mt19937 rng(seed);
  // distinct ids, then null patterns drawn from a small set
  std::vector<int32_t> perm(p.num_blocks); for (int i = 0; i < p.num_blocks; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), rng);
  if ((uint64_t)n * G * k > (uint64_t)p.num_blocks) FAIL("pool too small for the test");
  std::vector<int32_t> ids(n * G * k);
  for (size_t i = 0; i < ids.size(); ++i) ids[i] = perm[i];
  std::vector<std::vector<uint8_t>> pats(n_patterns, std::vector<uint8_t>(G * k));
  for (auto& pt : pats) for (auto& x : pt) x = (rng() % 3) == 0;
  if (n_patterns > 1) std::fill(pats[1].begin(), pats[1].end(), 1);  // an all-null chunk
  if (!expect_grouped && n_patterns == 1) std::fill(pats[0].begin(), pats[0].end(), 0);  // no nulls
  std::vector<int32_t> tokv(n_tok_values);
  for (auto& t : tokv) t = rng() % (p.chunk_tokens + 1);
  if (n_tok_values > 1) tokv[0] = 0;
  std::vector<int32_t> toks(n);
  for (int c = 0; c < n; ++c) {
    const auto& pt = pats[rng() % n_patterns];
    for (uint64_t i = 0; i < G * k; ++i) if (pt[i]) ids[c * G * k + i] = -1;
    toks[c] = n_tok_values ? tokv[rng() % n_tok_values] : 0;
  }
  std::vector<void*> objp(n * O);
  std::map<uint64_t, std::pair<uint32_t,uint32_t>> obj_of;
  for (int c = 0; c < n; ++c) for (uint64_t o = 0; o < O; ++o) { uint64_t a = (1ull << 40) + (uint64_t)(c * O + o) * (1ull << 28); objp[c * O + o] = (void*)a; obj_of[a] = {(uint32_t)c, (uint32_t)o}; }
  hkv_chunk_batch b{}; b.n_chunks = n; b.block_ids = ids.data(); b.objects = objp.data(); b.chunk_tokens = n_tok_values ? toks.data() : nullptr;
  // plain launch
  hkv::WorkspaceLayout wl = hkv::workspace_layout(p.dev_layers.size(), p.items.size(), n, G, k, O);
  std::vector<uint8_t> tab(wl.total);
  memcpy(tab.data() + wl.layers_off, p.dev_layers.data(), p.dev_layers.size() * sizeof(hkv::DevLayer));
  memcpy(tab.data() + wl.items_off, p.items.data(), p.items.size() * 8);
  memcpy(tab.data() + wl.ids_off, ids.data(), ids.size() * 4);
  for (size_t i = 0; i < objp.size(); ++i) ((uint64_t*)(tab.data() + wl.objs_off))[i] = (uint64_t)objp[i];
  if (b.chunk_tokens) memcpy(tab.data() + wl.tokens_off, toks.data(), n * 4);
  std::vector<Op> want, got;
  if (ops_of(name, p, tab.data(), tab.size(), wl.items_off, p.items.size(), wl.ids_off, wl.objs_off, wl.tokens_off, b.chunk_tokens != nullptr, n, obj_of, &want)) return 1;
  if (!codec) {
    // DMA retrieve: every plain copy lies inside one run at the same offset on
    // both sides, and the runs move exactly the plain copies' bytes.
    const uint64_t pool_base = 1ull << 44;
    std::vector<hkv::DmaRun> runs;
    hkv::plan_dma_runs(p, b, pool_base, &runs);
    std::sort(runs.begin(), runs.end(), [](const hkv::DmaRun& x, const hkv::DmaRun& y) { return x.src < y.src; });
    uint64_t run_bytes = 0, op_bytes = 0;
    for (size_t i = 0; i < runs.size(); ++i) {
      run_bytes += runs[i].bytes;
      if (i && runs[i].src < runs[i - 1].src + runs[i - 1].bytes) FAIL("DMA runs overlap in the objects");
    }
    for (const Op& op : want) {
      const uint64_t dst = pool_base + std::get<0>(op), len = std::get<1>(op);
      const uint64_t src = (uint64_t)objp[std::get<2>(op) * O + std::get<3>(op)] + std::get<4>(op);
      auto it = std::upper_bound(runs.begin(), runs.end(), src, [](uint64_t v, const hkv::DmaRun& r) { return v < r.src; });
      if (it == runs.begin()) FAIL("a copy outside every DMA run");
      --it;
      if (src + len > it->src + it->bytes || dst - it->dst != src - it->src) FAIL("a copy not matched by its DMA run");
      op_bytes += len;
    }
    if (run_bytes != op_bytes) FAIL("DMA runs move %llu bytes, the copies %llu", (unsigned long long)run_bytes, (unsigned long long)op_bytes);
    printf("%-16s DMA: %zu runs for %zu copies (%llu bytes)\n", name, runs.size(), want.size(), (unsigned long long)run_bytes);
  }
  hkv::GroupedCall g;
  const bool grouped = hkv::plan_grouped_retrieve(p, b, &g);
  if (grouped != expect_grouped) FAIL("grouped = %d, expected %d (%zu classes)", grouped, expect_grouped, g.members.size());
  if (!grouped) { printf("%-16s codec %d: plain launch (%zu+ classes), %zu copies\n", name, codec, g.members.size(), want.size()); return 0; }
  const uint64_t need = std::max(wl.total, hkv::grouped_layout(p, hkv::kMaxCallGroups * p.items.size(), n).total);
  if (g.ws.total > need) FAIL("grouped tables larger than the workspace size");
  std::vector<uint8_t> gt(g.ws.total, 0xEE);
  hkv::fill_grouped_tables(p, b, g, gt.data());
  uint64_t launched = 0;
  for (const auto& L : g.launches) {
    if (ops_of(name, p, gt.data(), gt.size(), L.items_off, L.n_items, L.ids_off, L.objs_off, L.tokens_off, b.chunk_tokens != nullptr, L.n_chunks, obj_of, &got)) return 1;
    launched += L.n_items * L.n_chunks;
  }
  if (launched != g.launched_items) FAIL("launched item count");
  std::sort(want.begin(), want.end()); std::sort(got.begin(), got.end());
  if (want != got) FAIL("copies differ: %zu vs %zu", want.size(), got.size());
  printf("%-16s codec %d: %zu classes, %zu launches, items %llu -> %llu, %zu copies identical\n", name, codec, g.members.size(), g.launches.size(),
         (unsigned long long)(n * p.items.size()), (unsigned long long)launched, want.size());
  return 0;
}

int check_inline();
int main() {
  if (check_inline()) return 1;
  int bad = 0;
  for (int codec : {0, 1}) {
    bad |= check("tiny", {0,0,0,1}, 2, 16, 96, 2, 0, 64ull*16*576*2, 0, 1, codec, 12, 3, 2, 1, true);
    bad |= check("tiny_notok", {0,0,0,1}, 2, 16, 96, 2, 0, 64ull*16*576*2, 0, 1, codec, 12, 3, 0, 2, true);
    bad |= check("kl_tp1", kimi27(), 32, 128, 12288, 2, 1, 64ull<<30, 0, 1, codec, 40, 2, 2, 3, true);
    bad |= check("k3_tp8", k393(), 6, 128, 2304, 1, 0, 24ull<<30, 768, 1500, codec, 30, 3, 2, 4, true);
    bad |= check("k3_many", k393(), 6, 128, 2304, 1, 0, 24ull<<30, 768, 1500, codec, 60, 6, 5, 5, false);
    bad |= check("kl_tp1_whole", kimi27(), 32, 128, 12288, 2, 1, 64ull<<30, 0, 1, codec, 40, 1, 0, 6, false);
  }
  return bad;
}

// Inline tables: read back as the kernel reads them.
int check_inline() {
  const char* name = "inline";
  std::vector<uint8_t> m = kimi27();
  for (int codec : {0, 1}) for (int path : {0, 1}) {
    hkv_layout_desc desc{}; desc.model.n_layers = m.size(); desc.model.is_mla = m.data();
    desc.model.kda_heads=32; desc.model.kda_head_dim=128; desc.model.kda_state_bytes=4; desc.model.conv_dim=12288; desc.model.conv_kernel=4; desc.model.conv_bytes=2; desc.model.mla_width=576; desc.model.mla_bytes=2;
    desc.chunk_min_tokens=1; desc.path=path; desc.separate_object_groups=1; desc.pool_bytes=64ull<<30; desc.kda_codec=codec;
    hkv::Plan p; std::string err;
    if (hkv::make_plan(desc, &p, &err) != HKV_OK) FAIL("plan");
    const uint64_t G = p.n_kv_groups, k = p.blocks_per_chunk, O = p.n_obj_groups;
    int max_fit[2] = {0, 0};
    for (int tok = 0; tok < 2; ++tok) for (int n = 1; n <= 200; ++n) {
      std::vector<int32_t> ids(n * G * k); for (size_t i = 0; i < ids.size(); ++i) ids[i] = (int32_t)(i * 7 % p.num_blocks);
      std::vector<int32_t> toks(n); for (int c = 0; c < n; ++c) toks[c] = (c * 13) % (int)(p.chunk_tokens + 1);
      std::vector<void*> objp(n * O); for (size_t i = 0; i < objp.size(); ++i) objp[i] = (void*)((1ull << 40) + i * 4096);
      hkv_chunk_batch b{}; b.n_chunks = n; b.block_ids = ids.data(); b.objects = objp.data(); b.chunk_tokens = tok ? toks.data() : nullptr;
      hkv::InlineTables t; hkv::CopyArgs a{}; a.ids = (const int32_t*)1; a.objs = (const uint64_t*)1; a.chunk_tokens = (const int32_t*)1;
      const bool fit = hkv::pack_inline_tables(p, b, &t, &a);
      const uint64_t need = (n * G * k * 4 + 7) / 8 + n * O + (tok ? (n * 4 + 7) / 8 : 0);
      if (fit != (need <= hkv::kInlineWords)) FAIL("fit decision");
      if (!fit) { if (a.ids != (const int32_t*)1) FAIL("a changed without a fit"); continue; }
      max_fit[tok] = n;
      if (a.ids || a.objs || a.chunk_tokens) FAIL("pointers not cleared");
      const int32_t* rid = reinterpret_cast<const int32_t*>(t.words + a.inline_ids);
      const uint64_t* rob = t.words + a.inline_objs;
      const int32_t* rtk = reinterpret_cast<const int32_t*>(t.words + a.inline_tokens);
      if ((uint64_t)a.inline_objs + n * O > hkv::kInlineWords) FAIL("objects past the block");
      if (tok && (uint64_t)a.inline_tokens * 8 + n * 4 > hkv::kInlineWords * 8) FAIL("tokens past the block");
      if ((uint64_t)a.inline_ids * 8 + n * G * k * 4 > (uint64_t)a.inline_objs * 8) FAIL("ids overlap objects");
      for (size_t i = 0; i < ids.size(); ++i) if (rid[i] != ids[i]) FAIL("id %zu", i);
      for (size_t i = 0; i < objp.size(); ++i) if (rob[i] != (uint64_t)objp[i]) FAIL("obj %zu", i);
      if (tok) for (int c = 0; c < n; ++c) if (rtk[c] != toks[c]) FAIL("token %d", c);
    }
    printf("inline codec %d path %d: up to %d chunks inline (%d with token counts)\n", codec, path, max_fit[0], max_fit[1]);
  }
  return 0;
}
