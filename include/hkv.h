/*
 * hkv.h — chunk store/retrieve for hybrid KDA+MLA model caches on MI355X.
 *
 * The library moves a hybrid model's cache between a paged GPU pool (the
 * layout vLLM gives a model whose KDA linear-attention layers keep a
 * recurrent state and whose MLA layers keep per-token latent KV) and
 * contiguous chunk objects, one object per (chunk, object group):
 *
 *   store    : block-table gather, pool pages -> chunk objects;
 *   retrieve : scatter of chunk objects into newly allocated block ids.
 *
 * Pages are opaque bytes: the KDA state (recurrent heads x d x d plus conv
 * (conv_dim, kernel-1)) is one opaque page, as LMCache treats it ("Kimi-Linear"
 * and "Kimi K3" recipes, introduction; "Hybrid Attention Models",
 * Mamba / Linear-Attention Hybrids), so the copies are exact byte copies.
 *
 * Conventions for every call:
 *   - returns hkv_status: HKV_OK (0) or a negative error code; nothing aborts
 *     or throws; hkv_last_error() gives a message for the calling thread;
 *   - all validation happens on the host, synchronously, before any work is
 *     enqueued; a call that returns an error has enqueued nothing (except
 *     HKV_E_HIP, which reports a failure of the HIP runtime itself);
 *   - "HOST" arrays are read only during the call; "DEVICE" buffers must stay
 *     allocated until the stream has passed the enqueued work;
 *   - store/retrieve enqueue on the caller's stream and never synchronise it.
 *
 * Sizes are bytes unless stated; block ids are int32 in [0, num_blocks).
 */
#ifndef HKV_H
#define HKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hkv_status;

#define HKV_OK 0
#define HKV_E_ARG (-1)       /* malformed argument (NULL, negative count, bad enum) */
#define HKV_E_COVER (-2)     /* given N is not a multiple of 16 tokens or its MLA page
                                does not cover the KDA state page */
#define HKV_E_CHUNK (-3)     /* strict mode and the chunk minimum is not a multiple of N */
#define HKV_E_BATCH (-4)     /* max_num_batched_tokens outside the allowed range */
#define HKV_E_POOL (-5)      /* the pool holds no whole block (or more than INT32_MAX) */
#define HKV_E_RANGE (-6)     /* a block id outside [0, num_blocks) */
#define HKV_E_ALIAS (-7)     /* a retrieve target id repeated in one call, or two buffers
                                of one call overlap */
#define HKV_E_ALIGN (-8)     /* pool, object or workspace pointer not 16-byte aligned */
#define HKV_E_WORKSPACE (-9) /* workspace NULL or smaller than hkv_workspace_size() */
#define HKV_E_HIP (-10)      /* the HIP runtime reported an error (see hkv_last_error) */
#define HKV_E_CAPTURE (-11)  /* the stream is capturing and the call cannot be captured
                                (see hkv_store_chunks) */

/* One rank's model shapes.  KDA state shapes are PER RANK: heads and conv_dim
 * are already divided by the TP degree, because the KDA state is sharded
 * across TP ranks while the MLA cache is replicated ("Kimi-Linear" recipe,
 * Note; vLLM hybrid KV-cache blog, section 2.1 gives the two state shapes). */
typedef struct hkv_model {
  int32_t n_layers;        /* number of decoder layers, >= 1 */
  const uint8_t* is_mla;   /* HOST [n_layers], model order: 1 = MLA layer, 0 = KDA layer */
  int32_t kda_heads;       /* recurrent state heads per rank */
  int32_t kda_head_dim;    /* d: the recurrent state is heads x d x d */
  int32_t kda_state_bytes; /* bytes per recurrent-state element (4 = fp32) */
  int32_t conv_dim;        /* conv state rows per rank */
  int32_t conv_kernel;     /* conv kernel size; the state keeps kernel-1 columns */
  int32_t conv_bytes;      /* bytes per conv-state element (2 = bf16) */
  int32_t mla_width;       /* values per token per MLA layer (kv_lora_rank + rope dim, 576) */
  int32_t mla_bytes;       /* bytes per MLA value (2 = bf16, 1 = fp8 e4m3) */
} hkv_model;

/* Unified block size N: the smallest multiple of 16 tokens whose MLA page
 * (N x mla_width x mla_bytes) is at least one rank's KDA state page
 * (heads x d x d x state_bytes + conv_dim x (conv_kernel-1) x conv_bytes).
 * Defined in "Hybrid Attention Models", Mamba / Linear-Attention Hybrids,
 * Step 1 (vLLM forces one block size across groups so the attention page
 * covers the state page) and the "Kimi-Linear" recipe, Note (N follows the
 * per-rank state).  A model without KDA layers gets N = 16.
 * align_tokens must be 16 (the only step this library supports; 0 = 16).
 * Errors: HKV_E_ARG (NULL pointers, non-positive shapes, align != 16). */
hkv_status hkv_unified_block_size(const hkv_model* model, int32_t align_tokens,
                                  int64_t* n_out);

/* Everything a layout needs. */
typedef struct hkv_layout_desc {
  hkv_model model;
  int64_t block_size;         /* N in tokens; 0 = derive with the rule above; nonzero
                                 must be a multiple of 16 covering the KDA page
                                 (else HKV_E_COVER) */
  int64_t chunk_min_tokens;   /* >= 1: the chunk size is the smallest multiple of N at or
                                 above it ("Kimi K3" recipe, Why these settings) */
  int32_t strict_chunk_multiple; /* 1: HKV_E_CHUNK unless chunk_min_tokens % N == 0 (the
                                 older rule, "Kimi-Linear" recipe, Why these settings) */
  int32_t path;               /* 0 = path A, shared tensors with the unified padded page
                                 (vLLM hybrid KV-cache blog, section 3.1);
                                 1 = path B, packed per-layer offset + block stride
                                 (same blog, section 3.2) */
  int32_t separate_object_groups; /* 1: KDA and MLA layers go to different objects;
                                 0: one object holds every layer ("Hybrid Attention
                                 Models", Object-group separation) */
  const int32_t* kv_group_of_layer; /* HOST [n_layers] KV-cache group of each layer, ids
                                 0..G-1 all used; NULL = default: the MLA layers form one
                                 group, the KDA layers in model order form
                                 ceil(n_kda/n_mla) contiguous groups of sizes differing
                                 by at most one, larger first (Mooncake K3 blog, "Flat
                                 KV"); KDA groups are numbered before the MLA group */
  uint64_t pool_bytes;        /* bytes of the pool the layout may use */
  int64_t max_num_batched_tokens; /* 0 = skip; else must be >= N, and < 2N unless
                                 object groups are separated (HKV_E_BATCH) ("Kimi-Linear"
                                 recipe, Why these settings; "Hybrid Attention Models",
                                 Step 2) */
  uint64_t tile_bytes;        /* 0 = default (4 KiB); else the largest span one
                                 workgroup copies: a multiple of 4096 up to 1 GiB.  A
                                 tuning knob: results do not depend on it */
  uint32_t max_workgroups;    /* 0 = one workgroup per tile; else the grid is capped at
                                 this many workgroups, each looping over tiles.  A
                                 tuning knob: results do not depend on it */
  int32_t kda_codec;          /* 0 = KDA pages are stored as opaque bytes (default);
                                 1 = INT8 codec of the recurrent state in objects, for
                                 inactive checkpoints (Mooncake K3 blog, Compressed
                                 Checkpoint Storage: per-channel INT8 for the recurrent
                                 state, the conv window at full precision).  A KDA page
                                 is read as the conv state (conv_dim x (kernel-1) x
                                 conv_bytes, a multiple of 16 bytes) followed by the fp32
                                 recurrent state (heads x d x d, d in {16, 32, 64, 128,
                                 256}); in an object it becomes the conv bytes verbatim,
                                 then int8 codes of every row of d values, then one fp32
                                 scale per row.  Per row: s = (largest finite |x|) / 127;
                                 q = round-half-even(x / s) clamped to [-127, 127], and 0
                                 for non-finite x or s == 0 (x / s an IEEE fp32 division);
                                 retrieve writes q * s in fp32, a NaN product (only from an
                                 object the encoder did not write) as 0x7FC00000.  Lossy:
                                 |x - q s| <= s / 2 for finite x.  Else HKV_E_ARG */
} hkv_layout_desc;

typedef struct hkv_layout hkv_layout; /* opaque; its plan is immutable after init; may be
                                         shared by threads.  The first store or retrieve
                                         on a device copies the plan's constant tables
                                         (layer placements and per-chunk work items, about
                                         115 KB at the Kimi-Linear shapes) into that
                                         device's memory, synchronously; they stay there
                                         until hkv_layout_destroy. */

/* Plans a layout.  Path A: every layer uses the unified page P = the largest
 * real page (the MLA page), smaller KDA pages are padded to it; slab s holds
 * the s-th layer of every KV group, pool_offset = s x num_blocks x P,
 * stride P, num_blocks = pool_bytes / (slabs x P).  Path B: inside a group
 * the layers' real pages are packed in model order (running offset), the
 * block stride is the largest group total, num_blocks = pool_bytes /
 * stride.  Object layout: layer-major in model order, then the k blocks of
 * the chunk, real page bytes only, no header; for MLA layers this is an
 * [L_obj][chunk_tokens][mla_width] array.
 * Defined by: the block size N ("Hybrid Attention Models", Mamba /
 * Linear-Attention Hybrids, Step 1; "Kimi-Linear" recipe, Note), the chunk
 * size rule ("Kimi K3" recipe, Why these settings), one block table per KV
 * group (vLLM hybrid KV-cache blog, section 2.2), the two pool layouts (same
 * blog, sections 3.1 and 3.2), the balanced KDA groups (Mooncake K3 blog,
 * "Flat KV") and the separate object groups ("Hybrid Attention Models",
 * Object-group separation).
 * Errors: HKV_E_ARG, HKV_E_COVER, HKV_E_CHUNK, HKV_E_BATCH, HKV_E_POOL.
 * On success *out owns heap memory released by hkv_layout_destroy. */
hkv_status hkv_layout_init(const hkv_layout_desc* desc, hkv_layout** out);

/* Releases a layout and its tables in device memory.  NULL is ignored.  The
 * caller must not destroy a layout while a call that uses it is running on
 * another thread or while work it enqueued has not finished. */
void hkv_layout_destroy(hkv_layout* layout);

typedef struct hkv_layout_info {
  int64_t block_size;        /* N (tokens) */
  int64_t chunk_tokens;      /* C (tokens), a multiple of N */
  int32_t blocks_per_chunk;  /* k = C / N */
  int32_t n_layers;
  int32_t n_kv_groups;       /* G */
  int32_t n_obj_groups;      /* O: 1 or 2 */
  int64_t num_blocks;        /* valid block ids are [0, num_blocks) */
  int32_t path;              /* 0 = A, 1 = B */
  int32_t n_slabs;           /* path A: tensors = largest group size; path B: 0 */
  uint64_t unified_page_bytes; /* path A: P; path B: 0 */
  uint64_t block_stride;     /* bytes between consecutive block ids of one layer */
  uint64_t pool_bytes_used;  /* bytes of the pool the layout addresses */
  uint64_t obj_bytes[2];     /* bytes of one chunk's object of each object group (0 if
                                unused) */
  uint64_t chunk_payload_bytes; /* obj_bytes[0] + obj_bytes[1]: bytes moved per chunk */
  int32_t kda_codec;         /* as in hkv_layout_desc */
} hkv_layout_info;

/* Copies the layout's summary.  Errors: HKV_E_ARG. */
hkv_status hkv_layout_info_get(const hkv_layout* layout, hkv_layout_info* out);

typedef struct hkv_layer_info {
  int32_t is_mla;
  int32_t kv_group;          /* index into the block table's group axis */
  int32_t obj_group;         /* which object of the chunk holds this layer */
  int32_t slot;              /* position inside its KV group (path A: its slab) */
  uint64_t page_bytes;       /* real bytes of one page (copied) */
  uint64_t reserved_bytes;   /* bytes reserved per block (path A: P, padding included) */
  uint64_t pool_offset;      /* byte offset of block 0's page in the pool */
  uint64_t stride;           /* bytes between the pages of consecutive block ids */
  uint64_t obj_offset;       /* byte offset of block j=0's page inside its object; block j
                                sits at obj_offset + j * obj_page_bytes */
  uint64_t obj_page_bytes;   /* bytes one page takes in an object: page_bytes, or the INT8
                                form of a KDA page under the codec */
} hkv_layer_info;

/* Copies one layer's placement.  Errors: HKV_E_ARG (bad layer index). */
hkv_status hkv_layer_info_get(const hkv_layout* layout, int32_t layer, hkv_layer_info* out);

/* A block-table entry that names no page.  With a token budget of 2N or
 * more a scheduler step spans several blocks and only its last block gets a
 * KDA snapshot ("Kimi-Linear" recipe, Why these settings), so a KDA group's
 * table can have holes; an MLA block past a partial chunk's last token has
 * no page either.  Store writes zeros in a null page's place in the object (a
 * missing state reads as zero, as the engine zeroes the initial state of a
 * miss: vLLM hybrid KV-cache blog, section 5.3); retrieve writes nothing for
 * it.  Null ids may repeat within a call. */
#define HKV_NULL_BLOCK (-1)

/* One call's chunks. */
typedef struct hkv_chunk_batch {
  int32_t n_chunks;          /* >= 0; 0 is a no-op */
  const int32_t* block_ids;  /* HOST [n_chunks][G][k]: chunk c's block ids in each KV
                                group (one block table per group, vLLM hybrid KV-cache
                                blog, section 2.2), or HKV_NULL_BLOCK */
  void* const* objects;      /* HOST [n_chunks][O] pointers the GPU can address (device
                                memory, or pinned host memory from hipHostMalloc), each
                                to obj_bytes[o] bytes, 16-byte aligned, pairwise disjoint
                                and disjoint from the pool */
  const int32_t* chunk_tokens; /* HOST [n_chunks] valid tokens per chunk (0..C), or NULL
                                when every chunk is whole.  A partial chunk (a tail
                                registered at a fine boundary: vLLM hybrid KV-cache blog,
                                section 6.3; Mooncake K3 blog, fine-grained partial hits)
                                carries in MLA page j the token rows [j*N, min(t,
                                (j+1)*N)) only; store zeroes the rest of that page's
                                object bytes and retrieve writes only those rows.  KDA
                                pages are whole or null. */
  int32_t engine;            /* HKV_ENGINE_KERNEL (0): the gather/scatter kernels.
                                HKV_ENGINE_DMA (1), retrieve only: the pages go by DMA
                                copies on the stream (hipMemcpyAsync), one per run of
                                pages that are contiguous in both the object and the pool
                                (a path B KV group's pages of one block are one run).
                                For chunk objects in pinned host memory this leaves the
                                host link's other direction and the compute units to a
                                concurrent store (LMCache keeps objects in a pinned host
                                L1: "Kimi-Linear" and "Kimi K3" recipes).  Not for INT8
                                layouts (the codec decodes in the scatter kernel) or
                                stores (they zero-fill object bytes): HKV_E_ARG. */
} hkv_chunk_batch;

#define HKV_ENGINE_KERNEL 0
#define HKV_ENGINE_DMA 1

/* Device workspace bytes needed by a call with up to max_chunks chunks: the
 * call's tables (layer placements, work items, block ids, object addresses,
 * token counts), with room for up to 8 per-class item lists.  A retrieve
 * with null ids or partial chunks whose chunks fall into at most 8 classes
 * (same null entries, same token count) launches once per class over only
 * the work items that write something.  Errors: HKV_E_ARG. */
hkv_status hkv_workspace_size(const hkv_layout* layout, int32_t max_chunks, size_t* bytes);

/* Store (gather): for every chunk c, layer l and block j < k, copies the
 * page_bytes(l) bytes at pool + pool_offset(l) + block_ids[c][g(l)][j] x
 * stride(l) to objects[c][o(l)] + obj_offset(l) + j x obj_page_bytes(l).
 * The source address is the page of a block id in the layer's pool view
 * (vLLM hybrid KV-cache blog, sections 3.1 and 3.2: a layer's pages sit at
 * its offset plus block id times its stride); the destination bytes are the
 * opaque pages of the chunk's object of that layer's object group ("Hybrid
 * Attention Models", Object-group separation; "Kimi-Linear" recipe: the KDA
 * state is one opaque page per block).
 * (obj_page_bytes = page_bytes, except KDA pages under kda_codec = 1, which
 * are written in their INT8 form).  Padding and group slack are never read.
 * The pool is not modified.  Under kda_codec = 1 the first object pointer's
 * memory type (hipPointerGetAttributes) picks the gather: pinned host memory
 * takes a form that writes each row's codes as one run, which the host link
 * carries better; the bytes written are the same either way.
 * pool: DEVICE, 16-byte aligned, pool_bytes_used long.  workspace: DEVICE,
 * 16-byte aligned, ws_bytes >= hkv_workspace_size(n_chunks); it is
 * overwritten and must not be used by another call until the stream passes
 * this one.  stream: a hipStream_t (NULL = the default stream).
 * The call's block ids, object addresses and token counts travel in the
 * kernel arguments when they fit in 3 KiB (up to 96 chunks at the
 * Kimi-Linear shapes), so such a call is a single kernel launch; a larger
 * call first copies them into the workspace from pinned staging on the
 * same stream.
 * Repeated source ids are allowed.  Null ids and partial chunks: see
 * HKV_NULL_BLOCK and hkv_chunk_batch.chunk_tokens.
 * Graph capture: while `stream` is capturing (hipStreamBeginCapture), a call
 * whose tables travel in the kernel arguments is captured as its single
 * launch, and a DMA retrieve as its copies; a replay moves the bytes the
 * buffers hold at replay time.  Any other call returns HKV_E_CAPTURE and
 * enqueues nothing: a larger call (its staged table copy would replay
 * whatever the staging slot holds later), and a layout's first call on a
 * device (it uploads the layout's tables synchronously).  Null ids and
 * partial chunks are then served by one launch over all work items.
 * Errors: HKV_E_ARG (also a chunk_tokens entry outside [0, C]), HKV_E_RANGE
 * (an id neither HKV_NULL_BLOCK nor in [0, num_blocks)), HKV_E_ALIAS (objects
 * overlap each other, the pool or the workspace), HKV_E_ALIGN,
 * HKV_E_WORKSPACE, HKV_E_CAPTURE, HKV_E_HIP (a HIP call failed;
 * hkv_last_error names it). */
hkv_status hkv_store_chunks(const hkv_layout* layout, const void* pool,
                            const hkv_chunk_batch* batch, void* workspace, size_t ws_bytes,
                            void* stream);

/* Retrieve (scatter): the inverse copy, objects -> pages of the given,
 * newly allocated block ids (the engine hands the connector fresh block ids
 * to load a hit into: "Kimi K3" recipe, AMD MI355X notes; the loaded state
 * becomes the request's initial state: vLLM hybrid KV-cache blog, section
 * 5.3; page addresses as for hkv_store_chunks, sections 3.1 and 3.2).  Writes exactly the real page bytes of the
 * addressed pages and nothing else (KDA padding, group slack and every other
 * block are left as they were; a null id writes nothing, and a partial chunk
 * writes only its valid MLA token rows).  Because all groups share one
 * block-id space, every non-null id of the call must be distinct
 * (HKV_E_ALIAS otherwise).
 * Same buffer and capture rules as hkv_store_chunks; objects are not
 * modified.
 * Errors: HKV_E_ARG, HKV_E_RANGE, HKV_E_ALIAS, HKV_E_ALIGN, HKV_E_WORKSPACE,
 * HKV_E_CAPTURE, HKV_E_HIP. */
hkv_status hkv_retrieve_chunks(const hkv_layout* layout, void* pool,
                               const hkv_chunk_batch* batch, void* workspace,
                               size_t ws_bytes, void* stream);

#define HKV_OP_STORE 0
#define HKV_OP_RETRIEVE 1

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): hkv_store_chunks
 * (op = HKV_OP_STORE) or hkv_retrieve_chunks (op = HKV_OP_RETRIEVE) with the
 * same kernels and the same bytes in the pool and objects, but no workspace
 * and no allocation.  It calls no hipMalloc, hipFree, hipHostMalloc or other
 * allocating routine, and uses none of the library's pinned staging.
 *   - The layout's constant tables live in a static device array of the
 *     library, 4 MiB per device (held from the first such call on a device
 *     until the process ends); a layout whose tables are larger (more than
 *     about 500,000 work items per chunk) gets HKV_E_WORKSPACE.
 *   - The array holds several layouts' tables at once, each in a range of
 *     its own (about 117 KB at the Kimi-Linear shapes, so some 35 such
 *     layouts).  A call whose layout's tables are not there copies them in
 *     from the layout's host memory (hipMemcpyAsync from pageable memory,
 *     which the HIP runtime moves through its own staging) and waits for
 *     `stream` to finish; later calls with that layout on that device
 *     enqueue without waiting.  When the array is full, the layout used
 *     least recently is dropped to make room, except layouts that a captured
 *     call has used.  hkv_layout_destroy frees the layout's ranges.
 *   - While `stream` is capturing, a copy-in is refused (HKV_E_CAPTURE,
 *     nothing enqueued): make one call with each layout on the device before
 *     capturing.  A captured call reads its layout's tables when the graph
 *     replays, so that layout stays in the array until it is destroyed (do
 *     not replay the graph after that); when such layouts fill the array, a
 *     call that needs room gets HKV_E_WORKSPACE.
 *   - The call's block ids, object addresses and token counts travel in
 *     kernel arguments: one launch per run of chunks that fits (up to 96
 *     chunks at the Kimi-Linear shapes), so a large call is several launches.
 *   - Every call on a device shares that device's array.  Calls that
 *     overlap on one device (other streams, other threads) race only when
 *     one of them copies a layout in over the range of a layout that the
 *     other is using (an eviction, with more layouts than fit): order such
 *     calls.
 *   - A retrieve with null ids or partial chunks runs one launch over every
 *     work item per run of chunks (no per-class launches); the bytes written
 *     are the same.
 * pool: DEVICE as for hkv_store_chunks (written only by a retrieve).
 * batch: as for hkv_store_chunks; engine must be HKV_ENGINE_KERNEL.
 * Host-side checks keep per-thread buffers between calls, so a call no
 * larger than the thread's earlier ones does not allocate host memory either.
 * Errors: HKV_E_ARG (also a bad op, the DMA engine, or a chunk whose ids and
 * object addresses alone exceed the kernel-argument block), HKV_E_RANGE,
 * HKV_E_ALIAS (objects overlap each other or the pool; repeated retrieve
 * ids), HKV_E_ALIGN, HKV_E_WORKSPACE (tables larger than the static array, or
 * no room beside the layouts that captured calls use), HKV_E_CAPTURE,
 * HKV_E_HIP. */
hkv_status hkv_move_chunks_noalloc(const hkv_layout* layout, int32_t op, void* pool,
                                   const hkv_chunk_batch* batch, void* stream);

/* ------------------------------------------------------------------------
 * Object identity.  Cached pages are byte-opaque, so an entry must never be
 * read back by an engine whose object format differs: other attention
 * backends or kernel block sizes ("Kimi-Linear", "Kimi K3" recipes and
 * "Hybrid Attention Models", Caveats).  Objects are told apart by cache
 * group, prefix hash and parallel configuration (Mooncake K3 blog, vLLM x
 * Mooncake: hybrid cache reuse across instances).
 *
 * All hashing uses mix64, the output function of SplitMix64 (Steele, Lea and
 * Flood, OOPSLA 2014):
 *   mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *             z *= 0x94D049BB133111EB; z ^= z >> 31.
 * and GAMMA = 0x9E3779B97F4A7C15.  All arithmetic is modulo 2^64.
 * ------------------------------------------------------------------------ */

/* 64-bit fingerprint of the chunk-object format: it changes whenever the
 * bytes of an object would mean something else, and only then.  It folds,
 * with f = mix64(f ^ w) from f = GAMMA, the words: 1 (format version), N,
 * k, n_layers, kda_heads, kda_head_dim, kda_state_bytes, conv_dim,
 * conv_kernel, conv_bytes, mla_width, mla_bytes, n_obj_groups, kda_codec, and
 * per layer in model order is_mla | obj_group << 1 | obj_page_bytes << 8.  The pool path,
 * pool size, KV grouping and tuning knobs do not enter it: they do not change
 * object bytes, so objects stored from a path A pool can be retrieved into a
 * path B pool of the same model.  Errors: HKV_E_ARG. */
hkv_status hkv_layout_fingerprint(const hkv_layout* layout, uint64_t* out);

/* Chained prefix hashes and object keys for one request (vLLM hybrid
 * KV-cache blog, section 6.3: hashes are computed per hash block and each
 * folds in the previous one, so the i-th hash fingerprints the whole prefix;
 * a coarse block's hash is the hash of its last fine sub-block).
 *
 *   tokens            HOST [n_tokens] token ids of the request, in order;
 *   hash_block_tokens h: a divisor of N (0 = N);
 *   root              H_0, e.g. 0 or the hash a parent prefix ended on;
 *   rank_tag          the caller's parallel configuration (e.g. tp_size << 32
 *                     | tp_rank), mixed into every key;
 *   prefix_hashes_out HOST [n_tokens / h] or NULL: H_1 .. H_(n_tokens/h);
 *   keys_out          HOST [n_chunks][O] or NULL; n_chunks = n_tokens / C
 *                     (whole chunks only; a trailing partial chunk has none),
 *                     at most max_chunks are written;
 *   n_chunks_out      the number of whole chunks (may exceed max_chunks).
 *
 * Definitions (t_j = tokens[(i-1)*h + j], j = 0..h-1, as uint32):
 *   content_i = fold of c = mix64(c ^ (t_j | j << 32)) over j from c = GAMMA
 *   H_i       = mix64((H_{i-1} ^ content_i) + GAMMA)
 *   prefix(c) = H_{(c+1) C / h}                       (the chunk's last fine block)
 *   key(c, o) = mix64(mix64(fingerprint ^ rank_tag) ^ (prefix(c) + (o+1) GAMMA))
 * Errors: HKV_E_ARG (NULL tokens with n_tokens > 0, h not dividing N,
 * negative counts). */
hkv_status hkv_chunk_keys(const hkv_layout* layout, const int32_t* tokens, int64_t n_tokens,
                          int32_t hash_block_tokens, uint64_t root, uint64_t rank_tag,
                          uint64_t* prefix_hashes_out, uint64_t* keys_out, int32_t max_chunks,
                          int64_t* n_chunks_out);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * pointer stays valid until the thread's next hkv_* call. */
const char* hkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HKV_H */
