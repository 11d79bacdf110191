// Layout planner: turns an hkv_layout_desc into byte placements for every
// layer, the chunk-object layout, and the device tables the copy kernels
// read.  Host-only C++; no HIP calls.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "hkv.h"
#include "hkv_device_tables.hpp"

namespace hkv {

struct LayerPlacement {
  int32_t is_mla = 0;
  int32_t kv_group = 0;
  int32_t obj_group = 0;
  int32_t slot = 0;            // position inside the KV group (path A: slab)
  uint64_t page = 0;           // real bytes
  uint64_t reserved = 0;       // bytes reserved per block id
  uint64_t pool_offset = 0;    // block 0's page
  uint64_t stride = 0;         // between block ids
  uint64_t obj_offset = 0;     // block j = 0 inside the object
  uint64_t obj_page = 0;       // bytes one page takes in an object
};

struct Plan {
  int64_t block_size = 0;      // N
  int64_t chunk_tokens = 0;    // C
  int32_t blocks_per_chunk = 0;  // k
  int64_t num_blocks = 0;
  int32_t n_kv_groups = 0;
  int32_t n_obj_groups = 0;
  int32_t path = 0;
  int32_t n_slabs = 0;
  uint64_t unified_page = 0;
  uint64_t block_stride = 0;
  uint64_t pool_used = 0;
  uint64_t obj_bytes[2] = {0, 0};
  std::vector<LayerPlacement> layers;
  // Per-rank model shapes: kda_heads, kda_head_dim, kda_state_bytes,
  // conv_dim, conv_kernel, conv_bytes, mla_width, mla_bytes.
  int64_t shapes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t kda_codec = 0;       // 1: INT8 codec of the KDA recurrent state in objects
  uint64_t conv_part = 0;      // bytes of the conv state at the start of a KDA page

  // Copy decomposition: every (layer, block j, tile s) of one chunk is one
  // work item; the same list repeats for every chunk of a call.
  uint64_t tile_bytes = 0;
  uint32_t codec_rows_per_item = 0;
  uint32_t max_workgroups = 0;
  std::vector<DevLayer> dev_layers;
  std::vector<uint64_t> items;  // packed WorkItem per item of one chunk
};

// N from the model alone (the unified-block-size rule with a 16-token step).
hkv_status unified_block_size(const hkv_model& m, int64_t* n_out, std::string* err);

// Full plan.  On error returns the status and sets *err.
hkv_status make_plan(const hkv_layout_desc& d, Plan* out, std::string* err);

// Object-format fingerprint and chained prefix hashes / object keys
// (definitions in include/hkv.h).  hkv_keys.cpp.
uint64_t object_fingerprint(const Plan& p);
hkv_status chunk_keys(const Plan& p, const int32_t* tokens, int64_t n_tokens, int32_t hash_block,
                      uint64_t root, uint64_t rank_tag, uint64_t* prefix_out, uint64_t* keys_out,
                      int32_t max_chunks, int64_t* n_chunks_out, std::string* err);

}  // namespace hkv
