// Object identity: the object-format fingerprint and per-request chained
// prefix hashes / object keys.  Definitions are stated in include/hkv.h.
//
// Sources: the recipes' and "Hybrid Attention Models"' Caveats (byte-opaque
// entries must not be shared across attention backends or block sizes);
// vLLM hybrid KV-cache blog, section 6.3 (chained fine-grained hashes, a
// coarse block taking its last fine sub-block's hash); Mooncake K3 blog, vLLM
// x Mooncake (objects told apart by cache group, prefix hash and parallel
// configuration).
#include <string>

#include "hkv_plan.hpp"

namespace hkv {
namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014).
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Content hash of one hash block: tokens with their position in the block.
uint64_t block_content(const int32_t* t, int32_t h) {
  uint64_t c = kGamma;
  for (int32_t j = 0; j < h; ++j)
    c = mix64(c ^ ((uint64_t)(uint32_t)t[j] | ((uint64_t)(uint32_t)j << 32)));
  return c;
}

}  // namespace

uint64_t object_fingerprint(const Plan& p) {
  uint64_t f = kGamma;
  auto fold = [&f](uint64_t w) { f = mix64(f ^ w); };
  fold(1);  // format version: layer-major, block-minor, real page bytes, no header
  fold((uint64_t)p.block_size);
  fold((uint64_t)p.blocks_per_chunk);
  fold((uint64_t)p.layers.size());
  for (int64_t v : p.shapes) fold((uint64_t)v);
  fold((uint64_t)p.n_obj_groups);
  fold((uint64_t)p.kda_codec);
  for (const LayerPlacement& x : p.layers)
    fold((uint64_t)x.is_mla | ((uint64_t)x.obj_group << 1) | (x.obj_page << 8));
  return f;
}

hkv_status chunk_keys(const Plan& p, const int32_t* tokens, int64_t n_tokens, int32_t hash_block,
                      uint64_t root, uint64_t rank_tag, uint64_t* prefix_out, uint64_t* keys_out,
                      int32_t max_chunks, int64_t* n_chunks_out, std::string* err) {
  const int64_t h = hash_block ? hash_block : p.block_size;
  if (n_tokens < 0 || max_chunks < 0 || !n_chunks_out || (n_tokens > 0 && !tokens)) {
    if (err) *err = "chunk_keys: bad counts or NULL pointers";
    return HKV_E_ARG;
  }
  if (h <= 0 || p.block_size % h != 0) {
    if (err) *err = "hash_block_tokens must divide the block size N";
    return HKV_E_ARG;
  }
  const int64_t n_fine = n_tokens / h;
  const int64_t fine_per_chunk = p.chunk_tokens / h;
  const int64_t n_chunks = n_tokens / p.chunk_tokens;
  const uint64_t id_seed = mix64(object_fingerprint(p) ^ rank_tag);
  uint64_t H = root;
  int64_t chunk = 0;
  for (int64_t i = 1; i <= n_fine; ++i) {
    H = mix64((H ^ block_content(tokens + (i - 1) * h, (int32_t)h)) + kGamma);
    if (prefix_out) prefix_out[i - 1] = H;
    if (i % fine_per_chunk == 0) {  // H is the hash of this chunk's last fine block
      if (keys_out && chunk < max_chunks)
        for (int32_t o = 0; o < p.n_obj_groups; ++o)
          keys_out[chunk * p.n_obj_groups + o] = mix64(id_seed ^ (H + (uint64_t)(o + 1) * kGamma));
      ++chunk;
    }
  }
  *n_chunks_out = n_chunks;
  return HKV_OK;
}

}  // namespace hkv
