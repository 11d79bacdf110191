// Tables the host uploads into the caller's workspace for every call, and
// the kernel argument block.  Shared by the host planner/launcher and the
// HIP kernels (plain structs, no HIP types).
#pragma once

#include <cstdint>

namespace hkv {

// One layer's placement as the kernels see it (48 bytes).
struct DevLayer {
  uint64_t pool_offset;  // page of block 0
  uint64_t stride;       // bytes between block ids
  uint64_t obj_offset;   // page j = 0 inside the object
  uint64_t page;         // real bytes of one page
  uint32_t kv_group;
  uint32_t obj_group;
  uint32_t row_bytes;    // MLA: bytes per token row (a partial chunk keeps whole rows);
                         // KDA: 0 (a state page is whole or null)
  uint32_t pad_;
};
static_assert(sizeof(DevLayer) == 48, "DevLayer layout");

// A work item of one chunk, packed in 64 bits: layer (16) | block j (16) |
// tile index inside the page (32).
inline constexpr uint64_t pack_item(uint32_t layer, uint32_t j, uint32_t tile) {
  return (uint64_t)(layer & 0xFFFFu) | ((uint64_t)(j & 0xFFFFu) << 16) | ((uint64_t)tile << 32);
}

// Kernel argument block (passed by value).
struct CopyArgs {
  uint8_t* pool;
  const DevLayer* layers;
  const uint64_t* items;   // [items_per_chunk]
  const int32_t* ids;      // [n_chunks][G][k]
  const uint64_t* objs;    // [n_chunks][O] device addresses
  const int32_t* chunk_tokens;  // [n_chunks] valid tokens, or nullptr: all chunks whole
  uint64_t total_items;    // n_chunks * items_per_chunk
  uint64_t block_tokens;   // N
  uint64_t tile_bytes;
  uint32_t items_per_chunk;
  uint32_t n_kv_groups;
  uint32_t blocks_per_chunk;
  uint32_t n_obj_groups;
};

// Workspace sections, each starting on a 256-byte boundary.
struct WorkspaceLayout {
  uint64_t layers_off, items_off, ids_off, objs_off, tokens_off, total;
};

inline constexpr uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

inline WorkspaceLayout workspace_layout(uint64_t n_layers, uint64_t n_items, uint64_t n_chunks,
                                        uint64_t G, uint64_t k, uint64_t O) {
  WorkspaceLayout w{};
  w.layers_off = 0;
  w.items_off = w.layers_off + align256(n_layers * sizeof(DevLayer));
  w.ids_off = w.items_off + align256(n_items * sizeof(uint64_t));
  w.objs_off = w.ids_off + align256(n_chunks * G * k * sizeof(int32_t));
  w.tokens_off = w.objs_off + align256(n_chunks * O * sizeof(uint64_t));
  w.total = w.tokens_off + align256(n_chunks * sizeof(int32_t));
  return w;
}

}  // namespace hkv
