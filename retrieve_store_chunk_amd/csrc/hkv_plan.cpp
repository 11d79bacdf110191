// Layout planner.  Host-only; sizes are computed in closed form with
// overflow checks.
//
// Sources for the rules:
//  - unified block size: "Hybrid Attention Models" (LMCache docs),
//    Mamba / Linear-Attention Hybrids, Step 1; "Kimi-Linear" recipe, Note;
//  - chunk size as the smallest multiple of N at or above a minimum: "Kimi K3"
//    recipe, Why these settings (LMCache-side); strict multiple: "Kimi-Linear"
//    recipe, Why these settings;
//  - token budget: "Kimi-Linear" recipe, Why these settings; "Hybrid Attention
//    Models", Step 2;
//  - KV-cache groups by spec, one block table each: vLLM hybrid KV-cache blog,
//    section 2.2; balanced KDA groups on shared slabs: Mooncake K3 blog, "Flat KV";
//  - path A (shared tensors, padded unified page) and path B (packed offsets,
//    shared block stride): vLLM hybrid KV-cache blog, sections 3.1 and 3.2;
//  - object groups: "Hybrid Attention Models", Object-group separation.
#include "hkv_plan.hpp"
#include "hkv_launch.hpp"

#include <algorithm>
#include <limits>

namespace hkv {
namespace {

constexpr int64_t kAlignTokens = 16;
constexpr uint64_t kDefaultTile = 4096;  // measured best on MI355X for both directions
constexpr uint64_t kMaxTile = 1ull << 30;

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

hkv_status fail(std::string* err, hkv_status st, const std::string& msg) {
  if (err) *err = msg;
  return st;
}

struct Sizes {
  int64_t kda_page = 0;   // one rank's opaque KDA state page
  int64_t tok_bytes = 0;  // MLA bytes per token
  int32_t n_kda = 0, n_mla = 0;
};

hkv_status model_sizes(const hkv_model& m, Sizes* s, std::string* err) {
  if (m.n_layers < 1 || m.is_mla == nullptr)
    return fail(err, HKV_E_ARG, "model needs n_layers >= 1 and an is_mla array");
  if (m.kda_heads < 1 || m.kda_head_dim < 1 || m.kda_state_bytes < 1 || m.conv_dim < 0 ||
      m.conv_kernel < 1 || m.conv_bytes < 1 || m.mla_width < 1 || m.mla_bytes < 1)
    return fail(err, HKV_E_ARG, "model shapes must be positive (conv_dim >= 0)");
  int64_t rec = 0, conv = 0;
  bool ok = mul_ok(m.kda_heads, m.kda_head_dim, &rec) && mul_ok(rec, m.kda_head_dim, &rec) &&
            mul_ok(rec, m.kda_state_bytes, &rec) &&
            mul_ok(m.conv_dim, (int64_t)m.conv_kernel - 1, &conv) &&
            mul_ok(conv, m.conv_bytes, &conv) && add_ok(rec, conv, &s->kda_page);
  if (!ok) return fail(err, HKV_E_ARG, "KDA state page size overflows");
  s->tok_bytes = (int64_t)m.mla_width * m.mla_bytes;
  for (int32_t l = 0; l < m.n_layers; ++l) (m.is_mla[l] ? s->n_mla : s->n_kda)++;
  return HKV_OK;
}

// Smallest positive multiple of 16 tokens whose MLA page covers `need` bytes.
int64_t covering_block_size(int64_t need, int64_t tok_bytes) {
  const int64_t step_bytes = kAlignTokens * tok_bytes;
  return std::max<int64_t>(1, ceil_div(need, step_bytes)) * kAlignTokens;
}

// Default grouping: the MLA layers are one group; the KDA layers, in model
// order, are cut into ceil(n_kda / n_mla) runs whose sizes differ by at most
// one (the first n_kda % runs runs are one longer).  KDA groups come first.
void default_grouping(const hkv_model& m, const Sizes& s, std::vector<int32_t>* group,
                      int32_t* n_groups) {
  int32_t runs = 0;
  if (s.n_kda > 0) runs = s.n_mla > 0 ? (s.n_kda + s.n_mla - 1) / s.n_mla : 1;
  std::vector<int32_t> run_len(runs, runs ? s.n_kda / runs : 0);
  for (int32_t r = 0; r < (runs ? s.n_kda % runs : 0); ++r) run_len[r]++;
  int32_t run = 0, left = runs ? run_len[0] : 0;
  for (int32_t l = 0; l < m.n_layers; ++l) {
    if (m.is_mla[l]) {
      (*group)[l] = runs;  // the attention group follows the KDA runs
      continue;
    }
    if (left == 0) left = run_len[++run];
    (*group)[l] = run;
    --left;
  }
  *n_groups = runs + (s.n_mla > 0 ? 1 : 0);
}

}  // namespace

hkv_status unified_block_size(const hkv_model& m, int64_t* n_out, std::string* err) {
  Sizes s;
  hkv_status st = model_sizes(m, &s, err);
  if (st != HKV_OK) return st;
  *n_out = covering_block_size(s.n_kda > 0 ? s.kda_page : 0, s.tok_bytes);
  return HKV_OK;
}

hkv_status make_plan(const hkv_layout_desc& d, Plan* p, std::string* err) {
  const hkv_model& m = d.model;
  Sizes s;
  hkv_status st = model_sizes(m, &s, err);
  if (st != HKV_OK) return st;
  if (d.path != 0 && d.path != 1) return fail(err, HKV_E_ARG, "path must be 0 (A) or 1 (B)");
  // The INT8 codec reads fp32 rows of head_dim values (a power of two from 16
  // to 256, so one row maps onto 4..64 lanes) after a conv part of whole
  // 16-byte units.
  const int64_t conv_part = (int64_t)m.conv_dim * (m.conv_kernel - 1) * m.conv_bytes;
  if (d.kda_codec != 0 && d.kda_codec != 1)
    return fail(err, HKV_E_ARG, "kda_codec must be 0 or 1");
  if (d.kda_codec == 1) {
    const int32_t hd = m.kda_head_dim;
    const bool pow2 = hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256;
    if (m.kda_state_bytes != 4 || !pow2 || conv_part % 16 != 0)
      return fail(err, HKV_E_ARG,
                  "the INT8 codec needs an fp32 recurrent state, head_dim in {16..256} (a "
                  "power of two) and a conv state of whole 16-byte units");
  }

  // Block size N.
  int64_t n = 0;
  if (d.block_size == 0) {
    n = covering_block_size(s.n_kda > 0 ? s.kda_page : 0, s.tok_bytes);
  } else {
    n = d.block_size;
    if (n < 0 || n % kAlignTokens != 0)
      return fail(err, HKV_E_COVER, "block_size must be a multiple of 16 tokens");
    int64_t mla_page = 0;
    if (!mul_ok(n, s.tok_bytes, &mla_page)) return fail(err, HKV_E_ARG, "MLA page overflows");
    if (s.n_kda > 0 && mla_page < s.kda_page)
      return fail(err, HKV_E_COVER, "block_size too small: the MLA page (" +
                                        std::to_string(mla_page) +
                                        " B) does not cover the KDA state page (" +
                                        std::to_string(s.kda_page) + " B)");
  }

  // Chunk size.
  if (d.chunk_min_tokens < 1) return fail(err, HKV_E_ARG, "chunk_min_tokens must be >= 1");
  if (d.strict_chunk_multiple && d.chunk_min_tokens % n != 0)
    return fail(err, HKV_E_CHUNK, "chunk size " + std::to_string(d.chunk_min_tokens) +
                                      " is not a multiple of N = " + std::to_string(n));
  const int64_t k = ceil_div(d.chunk_min_tokens, n);
  if (k > 0xFFFF) return fail(err, HKV_E_ARG, "more than 65535 blocks per chunk");

  // Token budget.
  if (d.max_num_batched_tokens != 0) {
    const int64_t b = d.max_num_batched_tokens;
    if (b < n || (!d.separate_object_groups && b >= 2 * n))
      return fail(err, HKV_E_BATCH, "max_num_batched_tokens must be >= N" +
                                        std::string(d.separate_object_groups ? "" : " and < 2N"));
  }

  p->block_size = n;
  p->blocks_per_chunk = (int32_t)k;
  const int64_t shapes[8] = {m.kda_heads, m.kda_head_dim, m.kda_state_bytes, m.conv_dim,
                             m.conv_kernel, m.conv_bytes, m.mla_width, m.mla_bytes};
  std::copy(shapes, shapes + 8, p->shapes);
  p->kda_codec = d.kda_codec;
  p->conv_part = (uint64_t)conv_part;
  p->chunk_tokens = k * n;
  p->path = d.path;

  const int32_t L = m.n_layers;
  if (L > 0xFFFF) return fail(err, HKV_E_ARG, "more than 65535 layers");
  p->layers.assign(L, LayerPlacement{});
  int64_t mla_page = 0;
  if (!mul_ok(n, s.tok_bytes, &mla_page)) return fail(err, HKV_E_ARG, "MLA page overflows");
  for (int32_t l = 0; l < L; ++l) {
    p->layers[l].is_mla = m.is_mla[l] ? 1 : 0;
    p->layers[l].page = (uint64_t)(m.is_mla[l] ? mla_page : s.kda_page);
  }

  // KV-cache groups.
  std::vector<int32_t> group(L, 0);
  int32_t G = 0;
  if (d.kv_group_of_layer == nullptr) {
    default_grouping(m, s, &group, &G);
  } else {
    for (int32_t l = 0; l < L; ++l) {
      const int32_t g = d.kv_group_of_layer[l];
      if (g < 0 || g >= L) return fail(err, HKV_E_ARG, "kv_group_of_layer out of range");
      group[l] = g;
      G = std::max(G, g + 1);
    }
    std::vector<char> used(G, 0);
    for (int32_t l = 0; l < L; ++l) used[group[l]] = 1;
    if (std::find(used.begin(), used.end(), 0) != used.end())
      return fail(err, HKV_E_ARG, "kv_group_of_layer leaves a group id unused");
  }
  p->n_kv_groups = G;
  std::vector<int32_t> members(G, 0);
  for (int32_t l = 0; l < L; ++l) {
    p->layers[l].kv_group = group[l];
    p->layers[l].slot = members[group[l]]++;
  }

  // Pool placement.
  int64_t per_block = 0;
  if (d.path == 0) {
    uint64_t P = 0;
    for (const auto& x : p->layers) P = std::max(P, x.page);
    const int32_t slabs = *std::max_element(members.begin(), members.end());
    if (!mul_ok((int64_t)P, slabs, &per_block)) return fail(err, HKV_E_ARG, "overflow");
    p->unified_page = P;
    p->block_stride = P;
    p->n_slabs = slabs;
  } else {
    std::vector<uint64_t> run(G, 0);
    for (auto& x : p->layers) {
      x.pool_offset = run[x.kv_group];
      run[x.kv_group] += x.page;
    }
    per_block = (int64_t)*std::max_element(run.begin(), run.end());
    p->unified_page = 0;
    p->block_stride = (uint64_t)per_block;
    p->n_slabs = 0;
  }
  const uint64_t nb = d.pool_bytes / (uint64_t)per_block;
  if (nb < 1 || nb > (uint64_t)std::numeric_limits<int32_t>::max())
    return fail(err, HKV_E_POOL, "the pool must hold between 1 and 2^31-1 blocks of " +
                                     std::to_string(per_block) + " B");
  p->num_blocks = (int64_t)nb;
  p->pool_used = nb * (uint64_t)per_block;
  for (auto& x : p->layers) {
    if (d.path == 0) {
      x.reserved = p->unified_page;
      x.stride = p->unified_page;
      x.pool_offset = (uint64_t)x.slot * nb * p->unified_page;
    } else {
      x.reserved = x.page;
      x.stride = p->block_stride;
    }
  }

  // Object groups and the object byte layout (layer-major, then block j).
  // Under the codec a KDA page takes conv part + rows codes + rows scales.
  const uint64_t codec_rows = (uint64_t)m.kda_heads * (uint64_t)m.kda_head_dim;
  const uint64_t codec_page = (uint64_t)conv_part + codec_rows * (uint64_t)m.kda_head_dim +
                              codec_rows * 4;
  const bool split = d.separate_object_groups && s.n_kda > 0 && s.n_mla > 0;
  p->n_obj_groups = split ? 2 : 1;
  for (auto& x : p->layers) {
    x.obj_group = split ? x.is_mla : 0;
    x.obj_page = (d.kda_codec == 1 && !x.is_mla) ? codec_page : x.page;
    x.obj_offset = p->obj_bytes[x.obj_group];
    p->obj_bytes[x.obj_group] += (uint64_t)k * x.obj_page;
  }

  // Copy decomposition.
  uint64_t tile = d.tile_bytes ? d.tile_bytes : kDefaultTile;
  if (tile % 4096 != 0 || tile > kMaxTile)
    return fail(err, HKV_E_ARG, "tile_bytes must be a multiple of 4096 up to 1 GiB");
  p->tile_bytes = tile;
  p->max_workgroups = d.max_workgroups;
  // A codec item covers as many rows as one tile of fp32 input holds, in
  // whole workgroup passes (at least one).
  const uint64_t row_in = 4 * (uint64_t)m.kda_head_dim;
  const uint64_t per_pass =
      d.kda_codec == 1 ? kCopyThreads / codec_lanes_per_row((uint32_t)m.kda_head_dim) : 1;
  p->codec_rows_per_item =
      (uint32_t)(std::max<uint64_t>(1, tile / (row_in * per_pass)) * per_pass);
  p->dev_layers.clear();
  p->items.clear();
  for (int32_t l = 0; l < L; ++l) {
    const auto& x = p->layers[l];
    const bool codec = d.kda_codec == 1 && !x.is_mla;
    DevLayer dl{};
    dl.pool_offset = x.pool_offset;
    dl.stride = x.stride;
    dl.obj_offset = x.obj_offset;
    dl.page = x.page;
    dl.obj_page = x.obj_page;
    dl.copy_bytes = codec ? (uint64_t)conv_part : x.page;
    dl.kv_group = (uint32_t)x.kv_group;
    dl.obj_group = (uint32_t)x.obj_group;
    dl.row_bytes = x.is_mla ? (uint32_t)s.tok_bytes : 0;
    dl.codec_rows = codec ? (uint32_t)codec_rows : 0;
    dl.head_dim = codec ? (uint32_t)m.kda_head_dim : 0;
    p->dev_layers.push_back(dl);
    const uint64_t tiles = (dl.copy_bytes + tile - 1) / tile;
    const uint64_t groups =
        codec ? (codec_rows + p->codec_rows_per_item - 1) / p->codec_rows_per_item : 0;
    if (tiles > 0x7FFFFFFFull || groups > 0x7FFFFFFFull)
      return fail(err, HKV_E_ARG, "too many tiles per page");
    for (int64_t j = 0; j < k; ++j) {
      for (uint64_t t = 0; t < tiles; ++t)
        p->items.push_back(pack_item(l, (uint32_t)j, (uint32_t)t, 0));
      for (uint64_t g = 0; g < groups; ++g)
        p->items.push_back(pack_item(l, (uint32_t)j, (uint32_t)g, 1));
    }
  }
  if (p->items.size() > 0xFFFFFFFFull) return fail(err, HKV_E_ARG, "too many tiles per chunk");
  return HKV_OK;
}

}  // namespace hkv
