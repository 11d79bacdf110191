// Per-call planning on the host side, no HIP: the grouped retrieve (the
// launches of a retrieve whose chunks fall into a few classes, same null ids
// and same token count, each over only the work items that write something),
// the packing of a small call's tables into the kernel arguments, and the
// copies of a DMA retrieve.
#pragma once

#include <cstdint>
#include <vector>

#include "hkv.h"
#include "hkv_device_tables.hpp"
#include "hkv_plan.hpp"

namespace hkv {

constexpr size_t kMaxCallGroups = 8;

// Workspace of a grouped call: the layer table, the classes' item lists
// (n_items_total in all), then the call's ids, object addresses and token
// counts in class order.
inline WorkspaceLayout grouped_layout(const Plan& p, uint64_t n_items_total, uint64_t n) {
  return workspace_layout(p.dev_layers.size(), n_items_total, n, (uint64_t)p.n_kv_groups,
                          (uint64_t)p.blocks_per_chunk, (uint64_t)p.n_obj_groups);
}

// One launch of a grouped retrieve: its tables' offsets in the workspace.
struct GroupLaunch {
  uint64_t items_off, n_items;         // item list
  uint64_t ids_off, objs_off, tokens_off;
  uint64_t n_chunks;
};

struct GroupedCall {
  WorkspaceLayout ws{};                // layout of the staged tables
  std::vector<GroupLaunch> launches;   // classes with something to write
  std::vector<std::vector<uint32_t>> members;  // chunks of each class
  std::vector<std::vector<uint64_t>> items;    // item list of each class
  uint64_t launched_items = 0;         // workgroups launched in all (one per item)
};

// Classifies the batch's chunks.  Returns false (use the plain launch) when
// there are more than kMaxCallGroups classes or fewer than a tenth of the
// items would go.
bool plan_grouped_retrieve(const Plan& p, const hkv_chunk_batch& b, GroupedCall* out);

// Writes the grouped call's tables (out->ws layout, ws.total bytes) to `h`.
void fill_grouped_tables(const Plan& p, const hkv_chunk_batch& b, const GroupedCall& g,
                         uint8_t* h);

// A DMA retrieve: the live bytes of every page as copies, each run of pages
// that are contiguous both in the object and in the pool merged into one.
struct DmaRun {
  uint64_t dst;    // pool address
  uint64_t src;    // object address
  uint64_t bytes;
};

// The runs of a retrieve of batch b into the pool at `pool` (in object order
// per chunk and object group).  Null pages give nothing; a partial chunk's
// MLA pages give their valid rows.
void plan_dma_runs(const Plan& p, const hkv_chunk_batch& b, uint64_t pool,
                   std::vector<DmaRun>* out);

// Packs the call's block ids, object addresses and token counts into `t` and
// sets a's inline offsets, if they fit in kInlineWords words; returns false
// (nothing written) otherwise.
bool pack_inline_tables(const Plan& p, const hkv_chunk_batch& b, InlineTables* t, CopyArgs* a);

}  // namespace hkv
