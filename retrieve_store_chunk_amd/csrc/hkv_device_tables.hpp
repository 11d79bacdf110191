// Tables the host uploads into the caller's workspace for every call, and
// the kernel argument block.  Shared by the host planner/launcher and the
// HIP kernels (plain structs, no HIP types).
#pragma once

#include <cstdint>

namespace hkv {

// One layer's placement as the kernels see it (80 bytes).
struct DevLayer {
  uint64_t pool_offset;  // page of block 0
  uint64_t stride;       // bytes between block ids
  uint64_t obj_offset;   // page j = 0 inside the object
  uint64_t page;         // real bytes of one pool page
  uint64_t obj_page;     // bytes one page takes in an object
  uint64_t copy_bytes;   // bytes copied verbatim: the page, or the conv part under the codec
  uint32_t kv_group;
  uint32_t obj_group;
  uint32_t row_bytes;    // MLA: bytes per token row (a partial chunk keeps whole rows);
                         // KDA: 0 (a state page is whole or null)
  uint32_t codec_rows;   // codec: rows of head_dim fp32 values (heads x head_dim); else 0
  uint32_t head_dim;     // codec: values per row
  uint32_t pad_[3];
};
static_assert(sizeof(DevLayer) == 80, "DevLayer layout");

// A work item of one chunk, packed in 64 bits: layer (16) | block j (16) |
// index (31) | kind (1).  Kind 0: verbatim tile `index` of the page's
// copy_bytes; kind 1: codec row group `index`.
inline constexpr uint64_t pack_item(uint32_t layer, uint32_t j, uint32_t index, uint32_t kind) {
  return (uint64_t)(layer & 0xFFFFu) | ((uint64_t)(j & 0xFFFFu) << 16) |
         ((uint64_t)(index & 0x7FFFFFFFu) << 32) | ((uint64_t)(kind & 1u) << 63);
}
inline constexpr uint32_t item_layer(uint64_t w) { return (uint32_t)(w & 0xFFFFu); }
inline constexpr uint32_t item_block(uint64_t w) { return (uint32_t)((w >> 16) & 0xFFFFu); }
inline constexpr uint32_t item_index(uint64_t w) { return (uint32_t)((w >> 32) & 0x7FFFFFFFu); }
inline constexpr uint32_t item_kind(uint64_t w) { return (uint32_t)(w >> 63); }

// The following are the per-item arithmetic of the copy kernels, shared with
// the host programs that replay it (constexpr functions compile for both).

// Bytes at the start of a verbatim span (a page, or the conv part of a codec
// page) that hold data: all `span` bytes, none for a null id (id < 0), and
// for an MLA page (row_bytes > 0) of a partial chunk with `tokens` valid
// tokens, the rows [j * block_tokens, tokens) that fall into block j.
inline constexpr uint64_t live_span_bytes(int32_t id, uint64_t span, uint32_t row_bytes,
                                          bool has_tokens, int64_t tokens, uint32_t j,
                                          uint64_t block_tokens) {
  if (id < 0) return 0;
  if (!has_tokens || row_bytes == 0) return span;
  int64_t rows = tokens - (int64_t)j * (int64_t)block_tokens;
  rows = rows < 0 ? 0 : (rows > (int64_t)block_tokens ? (int64_t)block_tokens : rows);
  return (uint64_t)rows * row_bytes;
}

// Tile s of a span: its offset, its length (tile_bytes, the last one
// shorter) and how many of its bytes hold data (`valid` from
// live_span_bytes); a store zero-fills the rest of the tile in the object.
struct TileSpan {
  uint64_t off;
  uint32_t bytes;
  uint32_t live;
};
inline constexpr TileSpan tile_span(uint64_t span, uint32_t s, uint64_t tile_bytes,
                                    uint64_t valid) {
  const uint64_t off = (uint64_t)s * tile_bytes;
  const uint64_t rest = span - off;
  const uint32_t bytes = (uint32_t)(rest < tile_bytes ? rest : tile_bytes);
  const uint32_t live = valid > off ? (uint32_t)(valid - off < bytes ? valid - off : bytes) : 0u;
  return TileSpan{off, bytes, live};
}

// Most 16-byte vectors a lane holds of a codec row.
constexpr uint32_t kCodecVecs = 2;

// Lanes that hold one recurrent-state row of head_dim fp32 values in a codec
// item: head_dim / (4 * kCodecVecs), kept within 4..16 (a row's lanes reduce
// with DPP inside one row of 16 lanes), so each lane holds
// head_dim / (4 * lanes) 16-byte vectors.  A workgroup of `threads` lanes
// takes threads / lanes rows a pass.
inline constexpr uint32_t codec_lanes_per_row(uint32_t head_dim) {
  return head_dim / (4 * kCodecVecs) < 4    ? 4
         : head_dim / (4 * kCodecVecs) > 16 ? 16
                                            : head_dim / (4 * kCodecVecs);
}

// In a codec row, lane `sub`'s v-th 16-byte vector of fp32 input (so the
// row's lanes read contiguous bytes per load); its 4 codes are the row's
// 4-byte code word of the same index.
inline constexpr uint32_t codec_input_vector(uint32_t sub, uint32_t v, uint32_t lanes) {
  return sub + v * lanes;
}

// Line-wide code stores (a store whose objects are in host memory): the
// lanes of a row first exchange code words so that lane `sub` holds words
// vecs * sub + i, i < vecs, of the row, then writes them with one store of
// 4 * vecs bytes; the row's codes leave as one contiguous run from one
// instruction.  Word w of a row sits, before the exchange, in lane
// w % lanes as its vector w / lanes (codec_input_vector).
inline constexpr uint32_t codec_line_word(uint32_t sub, uint32_t i, uint32_t vecs) {
  return sub * vecs + i;
}
inline constexpr uint32_t codec_word_lane(uint32_t w, uint32_t lanes) { return w % lanes; }
inline constexpr uint32_t codec_word_vector(uint32_t w, uint32_t lanes) { return w / lanes; }

// The work item that workgroup b of a grid of `grid` workgroups takes first
// (it then strides by `grid`).  Workgroup b runs on XCD b % xcds.
//   run == 0: XCD x takes one contiguous range of the items, so the
//             workgroups of an XCD sweep a narrow window of pages;
//   run > 0:  in each span of xcds runs of `run` items XCD x takes run x, in
//             order, so the XCDs work side by side on neighbouring runs; the
//             last partial span is split into one contiguous range per XCD.
// Either way the map is a bijection of [0, grid).
inline constexpr uint32_t xcd_first_item(uint32_t b, uint32_t grid, uint32_t run,
                                         uint32_t xcds) {
  const uint32_t x = b % xcds;
  if (run == 0) {
    const uint32_t q = grid / xcds, r = grid % xcds;
    return x * q + (x < r ? x : r) + b / xcds;
  }
  const uint32_t full = grid / (xcds * run) * (xcds * run);
  if (b < full) {
    const uint32_t j = b / xcds;
    return (j / run) * (xcds * run) + x * run + (j % run);
  }
  const uint32_t t = b - full, n = grid - full;
  const uint32_t q = n / xcds, r = n % xcds;
  return full + x * q + (x < r ? x : r) + t / xcds;
}

// Kernel argument block (passed by value).
struct CopyArgs {
  uint8_t* pool;
  const DevLayer* layers;
  const uint64_t* items;   // [items_per_chunk]
  const int32_t* ids;      // [n_chunks][G][k], or nullptr: in the InlineTables argument
  const uint64_t* objs;    // [n_chunks][O] device addresses, or nullptr: inline
  const int32_t* chunk_tokens;  // [n_chunks] valid tokens, or nullptr: inline (if has_tokens)
  uint64_t total_items;    // n_chunks * items_per_chunk
  uint64_t block_tokens;   // N
  uint64_t tile_bytes;
  uint32_t codec_rows_per_item;  // rows quantized by one kind-1 item (whole passes)
  uint32_t codec_head_dim;  // INT8 layouts: the KDA head_dim (selects the kernels); else 0
  uint32_t items_per_chunk;
  uint32_t n_kv_groups;
  uint32_t blocks_per_chunk;
  uint32_t n_obj_groups;
  uint32_t has_tokens;     // 0: every chunk is whole
  uint32_t inline_ids, inline_objs, inline_tokens;  // word offsets into InlineTables
  uint32_t codec_line_codes;  // INT8 store: run the line-code gather (objects in host memory)
};

// A call's block ids, object addresses and token counts, when they fit, travel
// in the kernel arguments (second argument, by value), so that a small call
// needs no copy ahead of its launch.
constexpr uint32_t kInlineWords = 384;  // 3 KiB
struct InlineTables {
  uint64_t words[kInlineWords];
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
