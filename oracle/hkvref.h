/*
 * hkvref — the CPU oracle for chunk store/retrieve of hybrid KDA+MLA caches.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * library (libhkv) never links it, never includes this header and shares no
 * source with it.
 *
 * What it computes, and where the pages define it:
 *   - unified block size N: "Hybrid Attention Models" (LMCache docs),
 *     Mamba / Linear-Attention Hybrids, Step 1; "Kimi-Linear" recipe, Note;
 *   - chunk size: "Kimi K3" recipe, Why these settings (LMCache-side): the
 *     chunk size is a minimum that is rounded up to a multiple of N; the
 *     older strict rule is in the "Kimi-Linear" recipe, Why these settings;
 *   - KV-cache groups: vLLM hybrid KV-cache blog, section 2.2; the balanced
 *     split of the KDA layers: Mooncake K3 blog, "Flat KV";
 *   - pool path A (shared tensor, unified padded page) and path B (packed,
 *     per-layer offset + shared block stride): vLLM hybrid KV-cache blog,
 *     sections 3.1 and 3.2;
 *   - object groups: "Hybrid Attention Models", Object-group separation;
 *   - the optional INT8 codec of inactive KDA states: Mooncake K3 blog,
 *     Compressed Checkpoint Storage;
 *   - store/retrieve: one memcpy per (chunk, layer, block) page.
 *
 * Every function returns 0 on success or a negative status code (the same
 * numeric codes as the product library, so tests can compare error
 * behaviour).  Nothing aborts.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every function here is
 * pinned; none is "parity unpinned".
 */
#ifndef HKVREF_H
#define HKVREF_H

#include <stdint.h>

#define HKVREF_OK 0
#define HKVREF_E_ARG (-1)
#define HKVREF_E_COVER (-2)
#define HKVREF_E_CHUNK (-3)
#define HKVREF_E_BATCH (-4)
#define HKVREF_E_POOL (-5)
#define HKVREF_E_RANGE (-6)
#define HKVREF_E_ALIAS (-7)

typedef struct hkvref_layout hkvref_layout;

/* Bytes of one rank's KDA state page: fp32-or-other recurrent state
 * heads x d x d plus the conv state conv_dim x (kernel-1). */
int64_t hkvref_kda_page_bytes(int32_t heads, int32_t head_dim, int32_t state_bytes,
                              int32_t conv_dim, int32_t conv_kernel, int32_t conv_bytes);

/* Smallest positive multiple of `align` tokens whose MLA page
 * (tokens x tok_bytes) is at least kda_page bytes. */
int hkvref_unified_block_size(int64_t kda_page, int64_t tok_bytes, int64_t align,
                              int64_t* n_out);

/* Negotiated chunk size (tokens) for a requested minimum. */
int hkvref_chunk_tokens(int64_t n, int64_t chunk_min, int32_t strict, int64_t* c_out);

/* Build a layout.  kv_group_of_layer may be NULL (default balanced split).
 * block_size 0 = derive N with the rule. max_batched 0 = skip that check. */
int hkvref_layout_init(int32_t n_layers, const uint8_t* is_mla,
                       int32_t heads, int32_t head_dim, int32_t state_bytes,
                       int32_t conv_dim, int32_t conv_kernel, int32_t conv_bytes,
                       int32_t mla_width, int32_t mla_bytes,
                       int64_t block_size, int64_t chunk_min, int32_t strict,
                       int32_t path, int32_t separate_objects,
                       const int32_t* kv_group_of_layer,
                       uint64_t pool_bytes, int64_t max_batched, int32_t kda_codec,
                       hkvref_layout** out);
void hkvref_layout_free(hkvref_layout* lay);

/* Summary: out[0]=N, [1]=C, [2]=k, [3]=num_blocks, [4]=n_layers,
 * [5]=G (KV groups), [6]=O (object groups), [7]=path, [8]=slabs (path A),
 * [9]=unified page P (path A, else 0), [10]=block stride (path B, else P),
 * [11]=obj_bytes[0], [12]=obj_bytes[1] (0 if O==1), [13]=bytes of the pool
 * the layout addresses, [14]=KDA codec (0 none, 1 INT8). */
int hkvref_layout_summary(const hkvref_layout* lay, int64_t out[15]);

/* Per layer: out[0]=is_mla, [1]=kv_group, [2]=obj_group, [3]=slab / index in
 * group, [4]=real page bytes, [5]=bytes reserved for it per block,
 * [6]=pool offset of block 0's page, [7]=stride between block ids,
 * [8]=offset of its block-0 page inside its object, [9]=bytes its page
 * takes in an object (the INT8 form for KDA layers under the codec). */
int hkvref_layer(const hkvref_layout* lay, int32_t layer, int64_t out[10]);

/* A block id that names no page: a missing KDA snapshot, or an MLA block
 * past a partial chunk's last token. */
#define HKVREF_NULL_BLOCK (-1)

/* Store: for each chunk c, copy every addressed page from `pool` into the
 * chunk's objects.  block_ids is [n_chunks][G][k] (ids or
 * HKVREF_NULL_BLOCK); chunk_tokens is [n_chunks] valid tokens per chunk
 * (0..C) or NULL for whole chunks; objects is [n_chunks][O] host pointers.
 * pool is a host buffer of at least summary[13] bytes.  Object bytes with no
 * data (null ids, MLA rows past the last valid token) are zeroed. */
int hkvref_store_chunks(const hkvref_layout* lay, const uint8_t* pool,
                        int32_t n_chunks, const int32_t* block_ids,
                        const int32_t* chunk_tokens, uint8_t* const* objects);

/* Retrieve: the inverse copy, objects -> pages at block_ids; null ids and
 * MLA rows past the last valid token are not written. */
int hkvref_retrieve_chunks(const hkvref_layout* lay, uint8_t* pool,
                           int32_t n_chunks, const int32_t* block_ids,
                           const int32_t* chunk_tokens, const uint8_t* const* objects);

/* The codec on one KDA page: encode = 1 turns a pool page (the layout's
 * page bytes) into its object form (object page bytes); encode = 0 the
 * reverse.  HKVREF_E_ARG if the layout has no codec. */
int hkvref_codec_page(const hkvref_layout* lay, int32_t encode, const uint8_t* in,
                      uint8_t* out);

/* Object-format fingerprint: mix64-fold (f = mix64(f ^ w), f0 = GAMMA) of
 * 1, N, k, n_layers, the eight per-rank shapes (heads, head_dim,
 * state_bytes, conv_dim, conv_kernel, conv_bytes, mla_width, mla_bytes),
 * n_obj_groups, codec, then per layer is_mla | obj_group << 1 |
 * object page bytes << 8. */
uint64_t hkvref_fingerprint(const hkvref_layout* lay);

/* Chained prefix hashes over hash blocks of h tokens (h divides N; 0 = N)
 * and one key per (whole chunk, object group).  prefix_out [n_tokens / h]
 * and keys_out [min(n_chunks, max_chunks)][O] may be NULL. */
int hkvref_chunk_keys(const hkvref_layout* lay, const int32_t* tokens, int64_t n_tokens,
                      int32_t hash_block, uint64_t root, uint64_t rank_tag,
                      uint64_t* prefix_out, uint64_t* keys_out, int32_t max_chunks,
                      int64_t* n_chunks_out);

#endif
