/*
 * hkvref.c — plain C oracle for chunk store/retrieve (TEST INFRASTRUCTURE).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  It is written from the pages' definitions in
 * the most direct form: straight loops over layers, one memcpy per page, no
 * blocking, no threads, no reordering.  It shares no source with the HIP
 * library.
 */
#include "hkvref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct hkvref_layout {
    int64_t n, c, k, num_blocks;
    int32_t n_layers, n_kv_groups, n_obj_groups, path, slabs;
    int64_t unified_page;  /* path A */
    int64_t block_stride;  /* path B (path A: = unified_page) */
    int64_t addressed_bytes;
    int64_t obj_bytes[2];
    int64_t shape[8]; /* heads, head_dim, state_bytes, conv_dim, conv_kernel, conv_bytes,
                         mla_width, mla_bytes */
    int32_t codec;      /* 0 = opaque KDA pages; 1 = INT8 recurrent-state codec */
    int64_t conv_part;  /* bytes of the conv state at the start of a KDA page */
    int64_t* obj_page;  /* bytes a layer's page takes in an object */
    int32_t* is_mla;
    int32_t* kv_group;
    int32_t* obj_group;
    int32_t* index_in_group;
    int64_t* page;
    int64_t* reserved;
    int64_t* pool_offset;
    int64_t* stride;
    int64_t* obj_offset;
};

/* One rank's KDA state page: the recurrent state (heads, d, d) and the conv
 * state (conv_dim, kernel-1), both already divided by the TP degree.
 * Source: vLLM hybrid KV-cache blog, section 2.1 (the two state shapes);
 * "Kimi-Linear" recipe, Note (the KDA state is sharded across TP ranks).
 * The opaque page is the plain sum of the two tensors' bytes ("Hybrid
 * Attention Models", Mamba / Linear-Attention Hybrids: the state is one
 * opaque page). */
int64_t hkvref_kda_page_bytes(int32_t heads, int32_t head_dim, int32_t state_bytes,
                              int32_t conv_dim, int32_t conv_kernel, int32_t conv_bytes)
{
    int64_t recurrent = (int64_t)heads * head_dim * head_dim * state_bytes;
    int64_t conv = (int64_t)conv_dim * (conv_kernel - 1) * conv_bytes;
    return recurrent + conv;
}

/* Unified block size: one block size for every KV-cache group, large enough
 * that an attention page is at least a KDA state page.  Source: "Hybrid
 * Attention Models", Step 1 (find N); "Kimi-Linear" recipe, Note (N is
 * chosen so the attention page covers the state page; it scales with the
 * per-rank state).  The step of 16 tokens is this library's reading. */
int hkvref_unified_block_size(int64_t kda_page, int64_t tok_bytes, int64_t align,
                              int64_t* n_out)
{
    int64_t n;
    if (tok_bytes <= 0 || align <= 0 || kda_page < 0 || n_out == NULL)
        return HKVREF_E_ARG;
    n = align; /* the smallest positive multiple */
    while (n * tok_bytes < kda_page)
        n += align;
    *n_out = n;
    return HKVREF_OK;
}

/* Chunk size.  Source: "Kimi K3" recipe, Why these settings (LMCache-side):
 * the requested chunk size is a minimum and the smallest multiple of N at
 * or above it is used; a lower minimum gives N.  Strict mode follows the
 * older statement ("Kimi-Linear" recipe, Why these settings) that a chunk
 * size which is not a multiple of N is an error. */
int hkvref_chunk_tokens(int64_t n, int64_t chunk_min, int32_t strict, int64_t* c_out)
{
    int64_t c;
    if (n <= 0 || chunk_min < 1 || c_out == NULL)
        return HKVREF_E_ARG;
    if (strict && chunk_min % n != 0)
        return HKVREF_E_CHUNK;
    c = n;
    while (c < chunk_min)
        c += n;
    *c_out = c;
    return HKVREF_OK;
}

static void layout_free_arrays(hkvref_layout* lay)
{
    free(lay->is_mla);
    free(lay->kv_group);
    free(lay->obj_group);
    free(lay->index_in_group);
    free(lay->page);
    free(lay->reserved);
    free(lay->pool_offset);
    free(lay->stride);
    free(lay->obj_offset);
    free(lay->obj_page);
}

void hkvref_layout_free(hkvref_layout* lay)
{
    if (lay == NULL)
        return;
    layout_free_arrays(lay);
    free(lay);
}

/* Default KV-cache grouping.  Layers with equal specs form a group (vLLM
 * hybrid KV-cache blog, section 2.2), and the KDA layers are split into
 * equal groups the size of the full-attention group so that one group of
 * each kind maps onto the same slabs (Mooncake K3 blog, "Flat KV": 69 KDA
 * layers in three groups of 23 plus the attention group on 24 slabs).
 * Reading: the MLA layers form one group of n_mla layers; the KDA layers, in
 * model order, form ceil(n_kda / n_mla) contiguous groups whose sizes differ
 * by at most one, larger groups first; KDA groups are numbered first, the
 * MLA group last. */
static void default_groups(int32_t n_layers, const int32_t* is_mla, int32_t* group,
                           int32_t* n_groups)
{
    int32_t n_mla = 0, n_kda = 0, m, base, rem, l, g, filled;
    for (l = 0; l < n_layers; l++) {
        if (is_mla[l])
            n_mla++;
        else
            n_kda++;
    }
    if (n_kda == 0) {
        m = 0;
    } else if (n_mla == 0) {
        m = 1;
    } else {
        m = (n_kda + n_mla - 1) / n_mla;
    }
    base = m > 0 ? n_kda / m : 0;
    rem = m > 0 ? n_kda % m : 0;
    g = 0;
    filled = 0;
    for (l = 0; l < n_layers; l++) {
        if (is_mla[l])
            continue;
        group[l] = g;
        filled++;
        if (filled == base + (g < rem ? 1 : 0)) {
            g++;
            filled = 0;
        }
    }
    for (l = 0; l < n_layers; l++) {
        if (is_mla[l])
            group[l] = m;
    }
    *n_groups = m + (n_mla > 0 ? 1 : 0);
}

int hkvref_layout_init(int32_t n_layers, const uint8_t* is_mla_in,
                       int32_t heads, int32_t head_dim, int32_t state_bytes,
                       int32_t conv_dim, int32_t conv_kernel, int32_t conv_bytes,
                       int32_t mla_width, int32_t mla_bytes,
                       int64_t block_size, int64_t chunk_min, int32_t strict,
                       int32_t path, int32_t separate_objects,
                       const int32_t* kv_group_of_layer,
                       uint64_t pool_bytes, int64_t max_batched, int32_t kda_codec,
                       hkvref_layout** out)
{
    hkvref_layout* lay;
    int64_t kda_page, tok_bytes, n, c, per_block;
    int32_t l, l2, g, o, n_kda = 0, n_mla = 0, rc;

    if (out == NULL || n_layers < 1 || is_mla_in == NULL || mla_width < 1 || mla_bytes < 1)
        return HKVREF_E_ARG;
    if (path != 0 && path != 1)
        return HKVREF_E_ARG;
    if (heads < 1 || head_dim < 1 || state_bytes < 1 || conv_dim < 0 || conv_kernel < 1 ||
        conv_bytes < 1)
        return HKVREF_E_ARG;
    /* The INT8 codec reads the recurrent state as fp32 rows of head_dim
     * values (16..256, a power of two) after a conv part of whole 16-byte
     * units. */
    if (kda_codec != 0 && kda_codec != 1)
        return HKVREF_E_ARG;
    if (kda_codec == 1 &&
        (state_bytes != 4 || (head_dim != 16 && head_dim != 32 && head_dim != 64 &&
                              head_dim != 128 && head_dim != 256) ||
         ((int64_t)conv_dim * (conv_kernel - 1) * conv_bytes) % 16 != 0))
        return HKVREF_E_ARG;

    lay = (hkvref_layout*)calloc(1, sizeof(*lay));
    if (lay == NULL)
        return HKVREF_E_ARG;
    lay->n_layers = n_layers;
    lay->path = path;
    lay->shape[0] = heads;
    lay->shape[1] = head_dim;
    lay->shape[2] = state_bytes;
    lay->shape[3] = conv_dim;
    lay->shape[4] = conv_kernel;
    lay->shape[5] = conv_bytes;
    lay->shape[6] = mla_width;
    lay->shape[7] = mla_bytes;
    lay->codec = kda_codec;
    lay->conv_part = (int64_t)conv_dim * (conv_kernel - 1) * conv_bytes;
    lay->is_mla = (int32_t*)calloc((size_t)n_layers, sizeof(int32_t));
    lay->kv_group = (int32_t*)calloc((size_t)n_layers, sizeof(int32_t));
    lay->obj_group = (int32_t*)calloc((size_t)n_layers, sizeof(int32_t));
    lay->index_in_group = (int32_t*)calloc((size_t)n_layers, sizeof(int32_t));
    lay->page = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    lay->reserved = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    lay->pool_offset = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    lay->stride = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    lay->obj_offset = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    lay->obj_page = (int64_t*)calloc((size_t)n_layers, sizeof(int64_t));
    if (!lay->is_mla || !lay->kv_group || !lay->obj_group || !lay->index_in_group ||
        !lay->page || !lay->reserved || !lay->pool_offset || !lay->stride || !lay->obj_offset ||
        !lay->obj_page) {
        hkvref_layout_free(lay);
        return HKVREF_E_ARG;
    }
    for (l = 0; l < n_layers; l++) {
        lay->is_mla[l] = is_mla_in[l] ? 1 : 0;
        if (lay->is_mla[l])
            n_mla++;
        else
            n_kda++;
    }

    /* N: the rule, or a given value checked against the same rule. */
    kda_page = hkvref_kda_page_bytes(heads, head_dim, state_bytes, conv_dim, conv_kernel,
                                     conv_bytes);
    tok_bytes = (int64_t)mla_width * mla_bytes;
    if (block_size == 0) {
        rc = hkvref_unified_block_size(n_kda > 0 ? kda_page : 0, tok_bytes, 16, &n);
        if (rc != HKVREF_OK) {
            hkvref_layout_free(lay);
            return rc;
        }
    } else {
        n = block_size;
        if (n < 0 || n % 16 != 0) {
            hkvref_layout_free(lay);
            return HKVREF_E_COVER;
        }
        if (n_kda > 0 && n * tok_bytes < kda_page) {
            hkvref_layout_free(lay);
            return HKVREF_E_COVER;
        }
    }
    lay->n = n;

    /* Chunk size and blocks per chunk. */
    rc = hkvref_chunk_tokens(n, chunk_min, strict, &c);
    if (rc != HKVREF_OK) {
        hkvref_layout_free(lay);
        return rc;
    }
    lay->c = c;
    lay->k = c / n;

    /* Scheduler budget ("Kimi-Linear" recipe, Why these settings; "Hybrid
     * Attention Models", Step 2): at least N; below 2N unless object groups
     * are separated. */
    if (max_batched != 0) {
        if (max_batched < n || (!separate_objects && max_batched >= 2 * n)) {
            hkvref_layout_free(lay);
            return HKVREF_E_BATCH;
        }
    }

    /* Real page bytes per layer.  MLA: (block_size, kv_lora_rank +
     * qk_rope_head_dim) values (vLLM hybrid KV-cache blog, section 4.2).
     * KDA: the opaque state page. */
    for (l = 0; l < n_layers; l++)
        lay->page[l] = lay->is_mla[l] ? n * tok_bytes : kda_page;

    /* KV-cache groups. */
    if (kv_group_of_layer == NULL) {
        default_groups(n_layers, lay->is_mla, lay->kv_group, &lay->n_kv_groups);
    } else {
        int32_t max_g = -1;
        for (l = 0; l < n_layers; l++) {
            if (kv_group_of_layer[l] < 0 || kv_group_of_layer[l] >= n_layers) {
                hkvref_layout_free(lay);
                return HKVREF_E_ARG;
            }
            lay->kv_group[l] = kv_group_of_layer[l];
            if (kv_group_of_layer[l] > max_g)
                max_g = kv_group_of_layer[l];
        }
        lay->n_kv_groups = max_g + 1;
        for (g = 0; g < lay->n_kv_groups; g++) {
            int32_t members = 0;
            for (l = 0; l < n_layers; l++)
                if (lay->kv_group[l] == g)
                    members++;
            if (members == 0) {
                hkvref_layout_free(lay);
                return HKVREF_E_ARG;
            }
        }
    }
    /* Position of each layer inside its group, in model order. */
    for (l = 0; l < n_layers; l++) {
        int32_t before = 0;
        for (l2 = 0; l2 < l; l2++)
            if (lay->kv_group[l2] == lay->kv_group[l])
                before++;
        lay->index_in_group[l] = before;
    }

    if (path == 0) {
        /* Path A (vLLM hybrid KV-cache blog, section 3.1): one page size for
         * every layer, the largest real page; smaller pages are padded to it.
         * Tensor s (a "slab") has page_size * num_blocks bytes and is shared
         * by the s-th layer of every group, so a block id maps to the same
         * offset block_id * page_size in each of them. */
        int64_t p = 0;
        int32_t slabs = 0;
        for (l = 0; l < n_layers; l++)
            if (lay->page[l] > p)
                p = lay->page[l];
        for (l = 0; l < n_layers; l++)
            if (lay->index_in_group[l] + 1 > slabs)
                slabs = lay->index_in_group[l] + 1;
        per_block = p * slabs;
        lay->num_blocks = (int64_t)(pool_bytes / (uint64_t)per_block);
        lay->unified_page = p;
        lay->block_stride = p;
        lay->slabs = slabs;
        for (l = 0; l < n_layers; l++) {
            lay->reserved[l] = p;
            lay->pool_offset[l] = (int64_t)lay->index_in_group[l] * lay->num_blocks * p;
            lay->stride[l] = p;
        }
        lay->addressed_bytes = lay->num_blocks * per_block;
    } else {
        /* Path B (vLLM hybrid KV-cache blog, section 3.2): inside a group the
         * layers' real pages are laid one after another (a running byte
         * offset); the block stride is the largest group total; num_blocks =
         * available bytes // block stride; each layer is the strided view
         * (offset, block_stride) of one shared backing. */
        int64_t stride = 0;
        for (g = 0; g < lay->n_kv_groups; g++) {
            int64_t byte_offset = 0;
            for (l = 0; l < n_layers; l++) {
                if (lay->kv_group[l] != g)
                    continue;
                lay->pool_offset[l] = byte_offset;
                byte_offset += lay->page[l];
            }
            if (byte_offset > stride)
                stride = byte_offset;
        }
        per_block = stride;
        lay->num_blocks = (int64_t)(pool_bytes / (uint64_t)per_block);
        lay->unified_page = 0;
        lay->block_stride = stride;
        lay->slabs = 0;
        for (l = 0; l < n_layers; l++) {
            lay->reserved[l] = lay->page[l];
            lay->stride[l] = stride;
        }
        lay->addressed_bytes = lay->num_blocks * per_block;
    }
    if (lay->num_blocks < 1 || lay->num_blocks > 2147483647LL) {
        hkvref_layout_free(lay);
        return HKVREF_E_POOL;
    }

    /* Object groups ("Hybrid Attention Models", Object-group separation):
     * separated, the KDA layers and the full-attention layers are stored as
     * different objects; otherwise one object holds every layer.  Reading:
     * object group 0 is the KDA group when there is one. */
    if (separate_objects && n_kda > 0 && n_mla > 0) {
        lay->n_obj_groups = 2;
        for (l = 0; l < n_layers; l++)
            lay->obj_group[l] = lay->is_mla[l] ? 1 : 0;
    } else {
        lay->n_obj_groups = 1;
        for (l = 0; l < n_layers; l++)
            lay->obj_group[l] = 0;
    }
    /* Object byte layout (reading): layer-major in model order, then the k
     * blocks of the chunk, real page bytes only, no header.  With the codec
     * a KDA page takes conv part + rows x head_dim codes + rows x 4 scale
     * bytes (rows = heads x head_dim). */
    for (l = 0; l < n_layers; l++) {
        int64_t rows = (int64_t)heads * head_dim;
        if (kda_codec == 1 && !lay->is_mla[l])
            lay->obj_page[l] = lay->conv_part + rows * head_dim + rows * 4;
        else
            lay->obj_page[l] = lay->page[l];
    }
    for (o = 0; o < 2; o++)
        lay->obj_bytes[o] = 0;
    for (l = 0; l < n_layers; l++) {
        o = lay->obj_group[l];
        lay->obj_offset[l] = lay->obj_bytes[o];
        lay->obj_bytes[o] += lay->k * lay->obj_page[l];
    }

    *out = lay;
    return HKVREF_OK;
}

int hkvref_layout_summary(const hkvref_layout* lay, int64_t out[15])
{
    if (lay == NULL || out == NULL)
        return HKVREF_E_ARG;
    out[0] = lay->n;
    out[1] = lay->c;
    out[2] = lay->k;
    out[3] = lay->num_blocks;
    out[4] = lay->n_layers;
    out[5] = lay->n_kv_groups;
    out[6] = lay->n_obj_groups;
    out[7] = lay->path;
    out[8] = lay->slabs;
    out[9] = lay->unified_page;
    out[10] = lay->block_stride;
    out[11] = lay->obj_bytes[0];
    out[12] = lay->n_obj_groups > 1 ? lay->obj_bytes[1] : 0;
    out[13] = lay->addressed_bytes;
    out[14] = lay->codec;
    return HKVREF_OK;
}

int hkvref_layer(const hkvref_layout* lay, int32_t layer, int64_t out[10])
{
    if (lay == NULL || out == NULL || layer < 0 || layer >= lay->n_layers)
        return HKVREF_E_ARG;
    out[0] = lay->is_mla[layer];
    out[1] = lay->kv_group[layer];
    out[2] = lay->obj_group[layer];
    out[3] = lay->index_in_group[layer];
    out[4] = lay->page[layer];
    out[5] = lay->reserved[layer];
    out[6] = lay->pool_offset[layer];
    out[7] = lay->stride[layer];
    out[8] = lay->obj_offset[layer];
    out[9] = lay->obj_page[layer];
    return HKVREF_OK;
}

/* ids[c][g][j] */
static int32_t block_id(const hkvref_layout* lay, const int32_t* ids, int32_t c, int32_t g,
                        int64_t j)
{
    return ids[((int64_t)c * lay->n_kv_groups + g) * lay->k + j];
}

static int check_ids(const hkvref_layout* lay, int32_t n_chunks, const int32_t* ids,
                     const int32_t* chunk_tokens, int unique)
{
    int64_t total = (int64_t)n_chunks * lay->n_kv_groups * lay->k, i;
    unsigned char* seen;
    for (i = 0; i < total; i++)
        if (ids[i] != HKVREF_NULL_BLOCK && (ids[i] < 0 || ids[i] >= lay->num_blocks))
            return HKVREF_E_RANGE;
    if (chunk_tokens != NULL)
        for (i = 0; i < n_chunks; i++)
            if (chunk_tokens[i] < 0 || chunk_tokens[i] > lay->c)
                return HKVREF_E_ARG;
    if (!unique)
        return HKVREF_OK;
    /* Retrieve writes every addressed page; the id space is shared by all
     * groups (vLLM hybrid KV-cache blog, sections 3.1 and 3.2), so distinct
     * ids are what keeps the written ranges apart.  Null ids write nothing. */
    seen = (unsigned char*)calloc((size_t)lay->num_blocks, 1);
    if (seen == NULL)
        return HKVREF_E_ARG;
    for (i = 0; i < total; i++) {
        if (ids[i] == HKVREF_NULL_BLOCK)
            continue;
        if (seen[ids[i]]) {
            free(seen);
            return HKVREF_E_ALIAS;
        }
        seen[ids[i]] = 1;
    }
    free(seen);
    return HKVREF_OK;
}

/* Bytes at the start of page j of layer l that hold data when the chunk has
 * t valid tokens.  An MLA page is N token rows of equal size (vLLM hybrid
 * KV-cache blog, section 4.2: (num_blocks, block_size, latent) view), so
 * block j holds rows for tokens [j*N, (j+1)*N) of the chunk.  A KDA page is a
 * whole state snapshot: all of it (a missing snapshot is a null id). */
static int64_t valid_bytes(const hkvref_layout* lay, int32_t l, int64_t j, int64_t t)
{
    int64_t rows;
    if (!lay->is_mla[l])
        return lay->page[l];
    rows = t - j * lay->n;
    if (rows < 0)
        rows = 0;
    if (rows > lay->n)
        rows = lay->n;
    return rows * (lay->page[l] / lay->n);
}

/* INT8 codec of the KDA recurrent state (Mooncake K3 blog, Compressed
 * Checkpoint Storage: inactive recurrent states are compressed to INT8 with
 * per-channel quantization parameters while the conv window keeps its
 * precision).  Readings: a channel is one row of head_dim values of the
 * (heads, d, d) state; s = (largest finite |x| of the row) / 127 in fp32;
 * q = round-half-even(x / s) clamped to [-127, 127]; non-finite x and rows
 * with s == 0 give q = 0; decoding gives q * s. */
static void encode_row(const float* x, int64_t d, int8_t* q, float* scale)
{
    float amax = 0.0f, s, v;
    int64_t i;
    for (i = 0; i < d; i++)
        if (isfinite(x[i]) && fabsf(x[i]) > amax)
            amax = fabsf(x[i]);
    s = amax / 127.0f;
    *scale = s;
    for (i = 0; i < d; i++) {
        if (s == 0.0f || !isfinite(x[i])) {
            q[i] = 0;
            continue;
        }
        v = rintf(x[i] / s);
        if (v > 127.0f)
            v = 127.0f;
        if (v < -127.0f)
            v = -127.0f;
        q[i] = (int8_t)v;
    }
}

/* Decoding is one fp32 product per value.  An object the encoder did not
 * write (a non-finite scale, code -128) can make it NaN; such a NaN is
 * written as the default quiet NaN 0x7FC00000, so the bytes do not depend on
 * which operand's payload a machine propagates. */
static void decode_row(const int8_t* q, float scale, int64_t d, float* x)
{
    const uint32_t qnan = 0x7FC00000u;
    int64_t i;
    for (i = 0; i < d; i++) {
        x[i] = (float)q[i] * scale;
        if (isnan(x[i]))
            memcpy(&x[i], &qnan, 4);
    }
}

/* A KDA page in codec form: the conv part verbatim, then the codes of every
 * row, then every row's scale.  The page is the conv state followed by the
 * recurrent state (the order of the two state shapes in vLLM hybrid KV-cache
 * blog, section 2.1). */
static void encode_page(const hkvref_layout* lay, const uint8_t* page, uint8_t* out)
{
    int64_t d = lay->shape[1], rows = lay->shape[0] * lay->shape[1], r;
    uint8_t* codes = out + lay->conv_part;
    uint8_t* scales = codes + rows * d;
    float* x = (float*)malloc((size_t)d * sizeof(float));
    int8_t* q = (int8_t*)malloc((size_t)d);
    memcpy(out, page, (size_t)lay->conv_part);
    for (r = 0; r < rows; r++) {
        float sc;
        memcpy(x, page + lay->conv_part + r * d * 4, (size_t)d * 4);
        encode_row(x, d, q, &sc);
        memcpy(codes + r * d, q, (size_t)d);
        memcpy(scales + r * 4, &sc, 4);
    }
    free(x);
    free(q);
}

static void decode_page(const hkvref_layout* lay, const uint8_t* in, uint8_t* page)
{
    int64_t d = lay->shape[1], rows = lay->shape[0] * lay->shape[1], r;
    const uint8_t* codes = in + lay->conv_part;
    const uint8_t* scales = codes + rows * d;
    float* x = (float*)malloc((size_t)d * sizeof(float));
    memcpy(page, in, (size_t)lay->conv_part);
    for (r = 0; r < rows; r++) {
        float sc;
        memcpy(&sc, scales + r * 4, 4);
        decode_row((const int8_t*)(codes + r * d), sc, d, x);
        memcpy(page + lay->conv_part + r * d * 4, x, (size_t)d * 4);
    }
    free(x);
}

int hkvref_codec_page(const hkvref_layout* lay, int32_t encode, const uint8_t* in,
                      uint8_t* out)
{
    if (lay == NULL || in == NULL || out == NULL || lay->codec != 1)
        return HKVREF_E_ARG;
    if (encode)
        encode_page(lay, in, out);
    else
        decode_page(lay, in, out);
    return HKVREF_OK;
}

/* Store: gather each chunk's pages out of the paged pool into its objects.
 * A page is copied as opaque bytes ("Kimi-Linear" recipe: LMCache treats the
 * KDA state as an opaque page; Caveats: the pages are byte-opaque).  Object
 * bytes with no data behind them (a null id, rows past a partial chunk's last
 * token) are written as zeros: a missing state reads as zero, as the engine
 * zeroes the initial state of a miss (vLLM hybrid KV-cache blog, section 5.3). */
int hkvref_store_chunks(const hkvref_layout* lay, const uint8_t* pool,
                        int32_t n_chunks, const int32_t* block_ids,
                        const int32_t* chunk_tokens, uint8_t* const* objects)
{
    int32_t c, l;
    int64_t j;
    int rc;
    if (lay == NULL || n_chunks < 0)
        return HKVREF_E_ARG;
    if (n_chunks == 0)
        return HKVREF_OK;
    if (pool == NULL || block_ids == NULL || objects == NULL)
        return HKVREF_E_ARG;
    rc = check_ids(lay, n_chunks, block_ids, chunk_tokens, 0);
    if (rc != HKVREF_OK)
        return rc;
    for (c = 0; c < n_chunks; c++) {
        int64_t t = chunk_tokens != NULL ? chunk_tokens[c] : lay->c;
        for (l = 0; l < lay->n_layers; l++) {
            uint8_t* obj = objects[(int64_t)c * lay->n_obj_groups + lay->obj_group[l]];
            for (j = 0; j < lay->k; j++) {
                int64_t id = block_id(lay, block_ids, c, lay->kv_group[l], j);
                uint8_t* dst = obj + lay->obj_offset[l] + j * lay->obj_page[l];
                int64_t v;
                if (id == HKVREF_NULL_BLOCK) {
                    memset(dst, 0, (size_t)lay->obj_page[l]);
                    continue;
                }
                if (lay->codec && !lay->is_mla[l]) {
                    encode_page(lay, pool + lay->pool_offset[l] + id * lay->stride[l], dst);
                    continue;
                }
                v = valid_bytes(lay, l, j, t);
                memcpy(dst, pool + lay->pool_offset[l] + id * lay->stride[l], (size_t)v);
                memset(dst + v, 0, (size_t)(lay->page[l] - v));
            }
        }
    }
    return HKVREF_OK;
}

/* Retrieve: scatter each chunk's objects back into the pages of the given
 * (newly allocated) block ids.  Only bytes that hold data are written: a null
 * id writes nothing, and a partial chunk's MLA pages get only their valid
 * token rows. */
int hkvref_retrieve_chunks(const hkvref_layout* lay, uint8_t* pool,
                           int32_t n_chunks, const int32_t* block_ids,
                           const int32_t* chunk_tokens, const uint8_t* const* objects)
{
    int32_t c, l;
    int64_t j;
    int rc;
    if (lay == NULL || n_chunks < 0)
        return HKVREF_E_ARG;
    if (n_chunks == 0)
        return HKVREF_OK;
    if (pool == NULL || block_ids == NULL || objects == NULL)
        return HKVREF_E_ARG;
    rc = check_ids(lay, n_chunks, block_ids, chunk_tokens, 1);
    if (rc != HKVREF_OK)
        return rc;
    for (c = 0; c < n_chunks; c++) {
        int64_t t = chunk_tokens != NULL ? chunk_tokens[c] : lay->c;
        for (l = 0; l < lay->n_layers; l++) {
            const uint8_t* obj = objects[(int64_t)c * lay->n_obj_groups + lay->obj_group[l]];
            for (j = 0; j < lay->k; j++) {
                int64_t id = block_id(lay, block_ids, c, lay->kv_group[l], j);
                if (id == HKVREF_NULL_BLOCK)
                    continue;
                if (lay->codec && !lay->is_mla[l]) {
                    decode_page(lay, obj + lay->obj_offset[l] + j * lay->obj_page[l],
                                pool + lay->pool_offset[l] + id * lay->stride[l]);
                    continue;
                }
                memcpy(pool + lay->pool_offset[l] + id * lay->stride[l],
                       obj + lay->obj_offset[l] + j * lay->obj_page[l],
                       (size_t)valid_bytes(lay, l, j, t));
            }
        }
    }
    return HKVREF_OK;
}

/* ------------------------------------------------------------------------
 * Object identity.  Cached pages are byte-opaque and must not be shared
 * across engines whose object format differs (the recipes' and "Hybrid
 * Attention Models"' Caveats); objects are told apart by cache group, prefix
 * hash and parallel configuration (Mooncake K3 blog, vLLM x Mooncake).
 * Hashes are chained per hash block, each folding in the previous one, and a
 * coarse block takes its last fine sub-block's hash (vLLM hybrid KV-cache
 * blog, section 6.3).  mix64 is SplitMix64's output function (Steele, Lea and
 * Flood, OOPSLA 2014).
 * ------------------------------------------------------------------------ */
#define HKVREF_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t ref_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t hkvref_fingerprint(const hkvref_layout* lay)
{
    uint64_t words[64];
    uint64_t f = HKVREF_GAMMA;
    int32_t i, l, n = 0;
    words[n++] = 1;
    words[n++] = (uint64_t)lay->n;
    words[n++] = (uint64_t)lay->k;
    words[n++] = (uint64_t)lay->n_layers;
    for (i = 0; i < 8; i++)
        words[n++] = (uint64_t)lay->shape[i];
    words[n++] = (uint64_t)lay->n_obj_groups;
    words[n++] = (uint64_t)lay->codec;
    for (i = 0; i < n; i++)
        f = ref_mix64(f ^ words[i]);
    for (l = 0; l < lay->n_layers; l++) {
        uint64_t w = (uint64_t)lay->is_mla[l] | ((uint64_t)lay->obj_group[l] << 1) |
                     ((uint64_t)lay->obj_page[l] << 8);
        f = ref_mix64(f ^ w);
    }
    return f;
}

int hkvref_chunk_keys(const hkvref_layout* lay, const int32_t* tokens, int64_t n_tokens,
                      int32_t hash_block, uint64_t root, uint64_t rank_tag,
                      uint64_t* prefix_out, uint64_t* keys_out, int32_t max_chunks,
                      int64_t* n_chunks_out)
{
    int64_t h = hash_block == 0 ? lay->n : hash_block;
    int64_t n_fine, n_chunks, i, j, c;
    uint64_t* H;
    uint64_t base;
    int32_t o;
    if (n_tokens < 0 || max_chunks < 0 || n_chunks_out == NULL ||
        (n_tokens > 0 && tokens == NULL))
        return HKVREF_E_ARG;
    if (h <= 0 || lay->n % h != 0)
        return HKVREF_E_ARG;
    n_fine = n_tokens / h;
    n_chunks = n_tokens / lay->c;
    /* H[0] = root; H[i] folds block i's content into H[i-1] */
    H = (uint64_t*)malloc((size_t)(n_fine + 1) * sizeof(uint64_t));
    if (H == NULL)
        return HKVREF_E_ARG;
    H[0] = root;
    for (i = 1; i <= n_fine; i++) {
        uint64_t content = HKVREF_GAMMA;
        for (j = 0; j < h; j++) {
            uint64_t t = (uint64_t)(uint32_t)tokens[(i - 1) * h + j];
            content = ref_mix64(content ^ (t | ((uint64_t)j << 32)));
        }
        H[i] = ref_mix64((H[i - 1] ^ content) + HKVREF_GAMMA);
        if (prefix_out != NULL)
            prefix_out[i - 1] = H[i];
    }
    /* chunk c ends on fine block (c+1) * C / h */
    base = ref_mix64(hkvref_fingerprint(lay) ^ rank_tag);
    if (keys_out != NULL) {
        for (c = 0; c < n_chunks && c < max_chunks; c++) {
            uint64_t prefix = H[(c + 1) * lay->c / h];
            for (o = 0; o < lay->n_obj_groups; o++)
                keys_out[c * lay->n_obj_groups + o] =
                    ref_mix64(base ^ (prefix + (uint64_t)(o + 1) * HKVREF_GAMMA));
        }
    }
    free(H);
    *n_chunks_out = n_chunks;
    return HKVREF_OK;
}
