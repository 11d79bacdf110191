// Grouped retrieve (see hkv_groups.hpp).  A retrieve writes nothing for a
// null page and nothing past a partial chunk's last valid row, yet the
// per-chunk item list launches a workgroup for every tile of every page.
#include "hkv_groups.hpp"

#include <cstring>
#include <map>

namespace hkv {

bool plan_grouped_retrieve(const Plan& p, const hkv_chunk_batch& b, GroupedCall* out) {
  const uint64_t n = (uint64_t)b.n_chunks;
  const uint64_t G = (uint64_t)p.n_kv_groups, k = (uint64_t)p.blocks_per_chunk;
  const uint64_t per_chunk = p.items.size();
  const int32_t* ids = b.block_ids;
  *out = GroupedCall{};
  // Class of each chunk: which (group, j) ids are null, and its token count.
  std::map<std::vector<int32_t>, size_t> class_of;
  std::vector<std::vector<int32_t>> signature;
  for (uint64_t c = 0; c < n; ++c) {
    std::vector<int32_t> sig(G * k + 1);
    for (uint64_t i = 0; i < G * k; ++i) sig[i] = ids[c * G * k + i] == HKV_NULL_BLOCK;
    sig[G * k] = b.chunk_tokens ? b.chunk_tokens[c] : -1;
    auto it = class_of.find(sig);
    if (it == class_of.end()) {
      if (out->members.size() == kMaxCallGroups) return false;
      it = class_of.emplace(sig, out->members.size()).first;
      out->members.emplace_back();
      signature.push_back(sig);
    }
    out->members[it->second].push_back((uint32_t)c);
  }
  // Each class keeps the items of its non-null pages that write at least a
  // byte, the same test as the kernel's live bytes.
  out->items.resize(out->members.size());
  uint64_t n_items_total = 0;
  for (size_t g = 0; g < out->members.size(); ++g) {
    const std::vector<int32_t>& sig = signature[g];
    const bool has_tokens = sig[G * k] >= 0;
    for (const uint64_t w : p.items) {
      const uint32_t j = item_block(w);
      const DevLayer& L = p.dev_layers[item_layer(w)];
      if (sig[L.kv_group * k + j]) continue;  // a null page
      if (item_kind(w) == 0) {
        // the kernel's own tile arithmetic (any non-null id writes the same bytes)
        const TileSpan ts = tile_span(
            L.copy_bytes, item_index(w), p.tile_bytes,
            live_span_bytes(0, L.copy_bytes, L.row_bytes, has_tokens, sig[G * k], j,
                            (uint64_t)p.block_size));
        if (ts.live == 0) continue;  // past the valid rows
      }
      out->items[g].push_back(w);
    }
    out->launched_items += out->members[g].size() * out->items[g].size();
    n_items_total += out->items[g].size();
  }
  if (out->launched_items * 10 > n * per_chunk * 9) return false;
  out->ws = grouped_layout(p, n_items_total, n);
  const uint64_t O = (uint64_t)p.n_obj_groups;
  uint64_t item_at = 0, chunk_at = 0;
  for (size_t g = 0; g < out->members.size(); ++g) {
    const uint64_t ng = out->members[g].size(), ni = out->items[g].size();
    if (ni > 0)
      out->launches.push_back({out->ws.items_off + item_at * sizeof(uint64_t), ni,
                               out->ws.ids_off + chunk_at * G * k * sizeof(int32_t),
                               out->ws.objs_off + chunk_at * O * sizeof(uint64_t),
                               out->ws.tokens_off + chunk_at * sizeof(int32_t), ng});
    item_at += ni;
    chunk_at += ng;
  }
  return true;
}

void fill_grouped_tables(const Plan& p, const hkv_chunk_batch& b, const GroupedCall& g,
                         uint8_t* h) {
  const uint64_t G = (uint64_t)p.n_kv_groups, k = (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  std::memcpy(h + g.ws.layers_off, p.dev_layers.data(), p.dev_layers.size() * sizeof(DevLayer));
  uint64_t* it = reinterpret_cast<uint64_t*>(h + g.ws.items_off);
  int32_t* id = reinterpret_cast<int32_t*>(h + g.ws.ids_off);
  uint64_t* ob = reinterpret_cast<uint64_t*>(h + g.ws.objs_off);
  int32_t* tk = reinterpret_cast<int32_t*>(h + g.ws.tokens_off);
  for (size_t c = 0; c < g.members.size(); ++c) {
    // (a class may have no items: memcpy from an empty vector's null data
    // pointer is undefined even for zero bytes)
    if (!g.items[c].empty())
      std::memcpy(it, g.items[c].data(), g.items[c].size() * sizeof(uint64_t));
    it += g.items[c].size();
    for (const uint32_t ch : g.members[c]) {
      std::memcpy(id, b.block_ids + (uint64_t)ch * G * k, G * k * sizeof(int32_t));
      id += G * k;
      for (uint64_t o = 0; o < O; ++o)
        *ob++ = reinterpret_cast<uintptr_t>(b.objects[(uint64_t)ch * O + o]);
      if (b.chunk_tokens) *tk++ = b.chunk_tokens[ch];
    }
  }
}

bool pack_inline_tables(const Plan& p, const hkv_chunk_batch& b, InlineTables* t, CopyArgs* a) {
  const uint64_t n = (uint64_t)b.n_chunks;
  const uint64_t n_ids = n * (uint64_t)p.n_kv_groups * (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups;
  const uint64_t id_words = (n_ids * sizeof(int32_t) + 7) / 8, obj_words = n * O;
  const uint64_t tok_words = b.chunk_tokens ? (n * sizeof(int32_t) + 7) / 8 : 0;
  if (id_words + obj_words + tok_words > kInlineWords) return false;
  std::memset(t, 0, sizeof(*t));
  std::memcpy(t->words, b.block_ids, n_ids * sizeof(int32_t));
  for (uint64_t i = 0; i < n * O; ++i)
    t->words[id_words + i] = reinterpret_cast<uintptr_t>(b.objects[i]);
  if (b.chunk_tokens)
    std::memcpy(t->words + id_words + obj_words, b.chunk_tokens, n * sizeof(int32_t));
  a->ids = nullptr;
  a->objs = nullptr;
  a->chunk_tokens = nullptr;
  a->inline_ids = 0;
  a->inline_objs = (uint32_t)id_words;
  a->inline_tokens = (uint32_t)(id_words + obj_words);
  return true;
}

void plan_dma_runs(const Plan& p, const hkv_chunk_batch& b, uint64_t pool,
                   std::vector<DmaRun>* out) {
  out->clear();
  const uint64_t G = (uint64_t)p.n_kv_groups, k = (uint64_t)p.blocks_per_chunk;
  const uint64_t O = (uint64_t)p.n_obj_groups, N = (uint64_t)p.block_size;
  for (uint64_t c = 0; c < (uint64_t)b.n_chunks; ++c) {
    const int64_t t = b.chunk_tokens ? b.chunk_tokens[c] : (int64_t)(N * k);
    for (uint64_t o = 0; o < O; ++o) {
      const uint64_t obj = reinterpret_cast<uintptr_t>(b.objects[c * O + o]);
      bool open = false;
      DmaRun run{};
      for (size_t l = 0; l < p.layers.size(); ++l) {
        const LayerPlacement& x = p.layers[l];
        if ((uint64_t)x.obj_group != o) continue;
        for (uint64_t j = 0; j < k; ++j) {
          const int32_t id = b.block_ids[(c * G + (uint64_t)x.kv_group) * k + j];
          if (id == HKV_NULL_BLOCK) continue;
          // (the DMA engine serves layouts without the codec: a page is copied
          // whole, or an MLA page's valid token rows)
          const uint64_t live =
              live_span_bytes(id, x.page, x.is_mla ? (uint32_t)(x.page / N) : 0u,
                              b.chunk_tokens != nullptr, t, (uint32_t)j, N);
          if (live == 0) continue;
          const uint64_t src = obj + x.obj_offset + j * x.obj_page;
          const uint64_t dst = pool + x.pool_offset + (uint64_t)id * x.stride;
          if (open && run.src + run.bytes == src && run.dst + run.bytes == dst) {
            run.bytes += live;
          } else {
            if (open) out->push_back(run);
            run = {dst, src, live};
            open = true;
          }
        }
      }
      if (open) out->push_back(run);
    }
  }
}

}  // namespace hkv
