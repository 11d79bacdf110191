// The copy kernels' index arithmetic replayed on the host over real plan
// tables, through the same helpers the kernels call (item decode, live
// bytes, tile spans, codec lane map in hkv_device_tables.hpp): for every
// work item of a call, every lane's loads and stores (16-byte copy vectors,
// or a codec item's 16-byte row loads, 4-byte code words and row scale) stay
// inside their page, row and object, are aligned for their width, and every
// object byte is written exactly once.  The DPP partners of the codec's row
// reduction stay inside the row's lanes, and so do the lanes that hand over
// code words for line-wide code stores (holding the words they hand over).
// Layouts: the five workloads' shapes and small ones with head_dim 16..256,
// three tile sizes, with and without the INT8 codec, with and without null
// ids and partial chunks.
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>
#include "hkv_launch.hpp"
#include "hkv_plan.hpp"

static const uint32_t kThreads = hkv::kCopyThreads;
static std::vector<uint8_t> kimi27() { std::vector<uint8_t> v; for (int i=0;i<24;i++) v.push_back(i%4==3); v.push_back(0); v.push_back(0); v.push_back(1); return v; }
static std::vector<uint8_t> k393() { std::vector<uint8_t> v; for (int i=0;i<92;i++) v.push_back(i%4==3); v.push_back(1); return v; }

#define FAIL(...) do { printf("%s: ", name); printf(__VA_ARGS__); printf("\n"); return 1; } while (0)

int check(const char* name, std::vector<uint8_t> is_mla, int heads, int d, int conv, int mlab, int path, uint64_t pool, int64_t N, int64_t cmin, int n_chunks, uint64_t tile, int codec, bool nulls, bool line = false) {
  hkv_layout_desc desc{}; desc.model.n_layers = is_mla.size(); desc.model.is_mla = is_mla.data();
  desc.model.kda_heads=heads; desc.model.kda_head_dim=d; desc.model.kda_state_bytes=4; desc.model.conv_dim=conv; desc.model.conv_kernel=4; desc.model.conv_bytes=2; desc.model.mla_width=576; desc.model.mla_bytes=mlab;
  desc.block_size=N; desc.chunk_min_tokens=cmin; desc.path=path; desc.separate_object_groups=1; desc.pool_bytes=pool; desc.tile_bytes=tile; desc.kda_codec=codec;
  hkv::Plan p; std::string err;
  if (hkv::make_plan(desc, &p, &err) != HKV_OK) FAIL("plan error %s", err.c_str());
  const uint64_t G=p.n_kv_groups, k=p.blocks_per_chunk, O=p.n_obj_groups, ipc=p.items.size();
  std::vector<int32_t> ids(n_chunks*G*k);
  for (size_t i=0;i<ids.size();i++) ids[i] = (int32_t)((p.num_blocks - 1 - i) % p.num_blocks);
  std::vector<int32_t> toks(n_chunks);
  for (int c=0;c<n_chunks;c++) toks[c] = (int32_t)p.chunk_tokens;
  if (nulls) {
    for (size_t i=0;i<ids.size();i+=3) ids[i] = -1;
    for (int c=1;c<n_chunks;c++) toks[c] = (int32_t)((c * 977) % (p.chunk_tokens + 1));
  }
  // object bases: 256-aligned like a caching allocator's (the API checks 16)
  std::vector<std::vector<uint8_t>> cover(n_chunks*O);
  for (uint64_t c=0;c<(uint64_t)n_chunks;c++) for (uint64_t o=0;o<O;o++) cover[c*O+o].assign(p.obj_bytes[o], 0);
  uint64_t total = n_chunks*ipc, moved=0, codec_items=0;
  auto mark = [&](std::vector<uint8_t>& cv, uint64_t lo, uint64_t n) -> int {
    if (lo + n > cv.size()) return 1;
    for (uint64_t b=lo;b<lo+n;b++) { if (cv[b]) return 2; cv[b]=1; }
    return 0;
  };
  for (uint64_t item=0; item<total; item++) {
    uint32_t c = item/ipc, r = item - c*ipc; uint64_t w = p.items[r];
    const uint32_t l = hkv::item_layer(w), j = hkv::item_block(w), s = hkv::item_index(w);
    const uint32_t kind = hkv::item_kind(w);
    if (l >= p.dev_layers.size() || j >= k) FAIL("bad item");
    const hkv::DevLayer& L = p.dev_layers[l];
    int32_t id = ids[((uint64_t)c*G + L.kv_group)*k + j];
    auto& cv = cover[c*O + L.obj_group];
    const uint64_t obj_page = L.obj_offset + (uint64_t)j*L.obj_page;   // offset in the object
    if (obj_page + L.obj_page > cv.size()) FAIL("object page past object");
    if (kind) {
      codec_items++;
      const uint32_t dd = L.head_dim, rows = L.codec_rows;
      if (!dd || !rows || L.row_bytes) FAIL("codec item on a non-codec layer");
      const uint32_t lpr = hkv::codec_lanes_per_row(dd);
      if ((lpr != 4 && lpr != 8 && lpr != 16) || kThreads % lpr || dd % (4 * lpr)) FAIL("lanes per row %u", lpr);
      const uint32_t vecs = dd / (4 * lpr);
      if (vecs > 8) FAIL("vectors per lane %u", vecs);
      const uint32_t rpp = kThreads / lpr;     // rows per pass
      if (p.codec_rows_per_item % rpp) FAIL("rows per item not whole passes");
      const uint32_t r0 = s * p.codec_rows_per_item;
      const uint32_t r_end = std::min<uint32_t>(r0 + p.codec_rows_per_item, rows);
      if (r0 >= rows) FAIL("codec group past rows");
      const uint64_t codes = obj_page + L.copy_bytes, scales = codes + (uint64_t)rows*dd;
      if (scales + (uint64_t)rows*4 != obj_page + L.obj_page) FAIL("codec page size");
      if (L.copy_bytes + (uint64_t)rows*dd*4 != L.page) FAIL("pool page size");
      if (id < 0) {   // store zero-fills codes + scales of these rows
        if (mark(cv, codes + (uint64_t)r0*dd, (uint64_t)(r_end-r0)*dd)) FAIL("null codes");
        if (mark(cv, scales + (uint64_t)r0*4, (uint64_t)(r_end-r0)*4)) FAIL("null scales");
        continue;
      }
      const uint64_t rec = L.pool_offset + (uint64_t)id*L.stride + L.copy_bytes;
      for (uint32_t t=0;t<kThreads;t++) {
        const uint32_t sub = t & (lpr-1);
        // DPP reduction partners stay inside the lane's aligned group of lpr
        if ((t ^ 1u) / lpr != t / lpr || (t ^ 2u) / lpr != t / lpr) FAIL("quad swap leaves the row");
        if (lpr >= 8 && ((t & ~7u) | (7u - (t & 7u))) / lpr != t / lpr) FAIL("half mirror leaves the row");
        if (lpr >= 16 && ((t & ~15u) | (15u - (t & 15u))) / lpr != t / lpr) FAIL("mirror leaves the row");
        for (uint32_t rr = r0 + t/lpr; rr < r_end; rr += rpp) {
          for (uint32_t v = 0; v < vecs; v++) {
            const uint32_t vi = hkv::codec_input_vector(sub, v, lpr);
            const uint64_t x = rec + (uint64_t)rr*dd*4 + (uint64_t)vi*16;
            if (x % 16) FAIL("unaligned 16-B load");
            if (x < rec + (uint64_t)rr*dd*4 || x + 16 > rec + (uint64_t)(rr+1)*dd*4) FAIL("load leaves its row");
            if (x + 16 > L.pool_offset + (uint64_t)id*L.stride + L.page || x + 16 > p.pool_used) FAIL("load past page");
            moved += 16;
            if (line) continue;
            // the 4 codes of that vector: one 4-byte word of the row's codes
            const uint64_t q = codes + (uint64_t)rr*dd + (uint64_t)vi*4;
            if (q % 4) FAIL("unaligned code store");
            if (q < codes + (uint64_t)rr*dd || q + 4 > codes + (uint64_t)(rr+1)*dd) FAIL("code store leaves its row");
            if (int e = mark(cv, q, 4)) FAIL("code store %s", e==1?"overflow":"twice");
          }
          if (line) {
            // line-wide codes: lane sub collects words codec_line_word(sub, i) from the
            // lanes that hold them (inside the row's aligned lane group, as the vector
            // the kernel selects), then writes them with one 4*vecs-byte store
            if (vecs != 1 && vecs != 2 && vecs != 4) FAIL("line store width %u", vecs);
            const uint32_t slot = hkv::codec_word_vector(hkv::codec_line_word(sub, 0, vecs), lpr);
            for (uint32_t i = 0; i < vecs; i++) {
              const uint32_t w = hkv::codec_line_word(sub, i, vecs);
              const uint32_t src = (t & 63u) - sub + hkv::codec_word_lane(w, lpr);
              if (src / lpr != (t & 63u) / lpr) FAIL("word source leaves the row");
              if (hkv::codec_word_vector(w, lpr) != slot) FAIL("a lane's words span two vectors");
              if (hkv::codec_input_vector(src % lpr, slot, lpr) != w) FAIL("source does not hold word");
            }
            const uint64_t q = codes + (uint64_t)rr*dd + (uint64_t)hkv::codec_line_word(sub, 0, vecs)*4;
            if (q % (4*vecs)) FAIL("unaligned line store");
            if (q < codes + (uint64_t)rr*dd || q + 4*vecs > codes + (uint64_t)(rr+1)*dd) FAIL("line store leaves its row");
            if (int e = mark(cv, q, 4*vecs)) FAIL("line store %s", e==1?"overflow":"twice");
          }
          if (sub == 0) { if (int e = mark(cv, scales + (uint64_t)rr*4, 4)) FAIL("scale store %s", e==1?"overflow":"twice"); }
        }
      }
      continue;
    }
    const uint64_t span = L.copy_bytes;
    if ((uint64_t)s*p.tile_bytes >= span) FAIL("tile past span");
    const hkv::TileSpan ts = hkv::tile_span(span, s, p.tile_bytes,
        hkv::live_span_bytes(id, span, L.row_bytes, nulls, toks[c], j, (uint64_t)p.block_size));
    const uint64_t off = ts.off, bytes = ts.bytes, live = ts.live;
    if (live) {
      if (id < 0) FAIL("live bytes for a null id");
      uint64_t src = L.pool_offset + (uint64_t)id*L.stride + off;
      if (src + live > p.pool_used || src + live > L.pool_offset + (uint64_t)id*L.stride + L.page) FAIL("pool overflow");
    }
    if (int e = mark(cv, obj_page + off, bytes)) FAIL("tile %s", e==1?"overflow":"twice");
    moved += live;
  }
  for (auto& cv : cover) if (std::find(cv.begin(), cv.end(), 0) != cv.end()) FAIL("object byte not written");
  printf("%-12s codec %d%s nulls %d ok: %llu items (%llu per chunk, %llu codec), %llu live bytes, tile %llu, rows/item %u\n", name, codec, line ? " (line codes)" : "", (int)nulls, (unsigned long long)total, (unsigned long long)ipc, (unsigned long long)codec_items, (unsigned long long)moved, (unsigned long long)p.tile_bytes, p.codec_rows_per_item);
  return 0;
}
int main() {
  int bad = 0;
  // codec 2: the INT8 codec with line-wide code stores (objects in host memory)
  for (int codec : {0, 1, 2}) for (bool nulls : {false, true})
  for (uint64_t tile : {0ull, 8192ull, 1ull<<20}) {
    const int c = codec ? 1 : 0;
    const bool line = codec == 2;
    bad |= check("tiny", {0,0,0,1}, 2, 16, 96, 2, 0, 64ull*16*576*2, 0, 1, 16, tile, c, nulls, line);
    bad |= check("tiny_d256", {0,0,0,1}, 1, 256, 96, 2, 1, 1ull<<28, 0, 1, 4, tile, c, nulls, line);
    bad |= check("tiny_d32", {0,1,0,1}, 3, 32, 8, 2, 0, 1ull<<27, 0, 40, 5, tile, c, nulls, line);
    bad |= check("tiny_d64", {0,1,0}, 3, 64, 104, 2, 0, 1ull<<27, 0, 40, 5, tile, c, nulls, line);
    bad |= check("kl_tp2", kimi27(), 16, 128, 6144, 2, 0, 16ull<<30, 0, 1, 3, tile, c, nulls, line);
    bad |= check("kl_tp1", kimi27(), 32, 128, 12288, 2, 1, 64ull<<30, 0, 1, 3, tile, c, nulls, line);
    bad |= check("k3_tp8", k393(), 6, 128, 2304, 1, 0, 24ull<<30, 768, 1500, 2, tile, c, nulls, line);
  }
  return bad;
}
