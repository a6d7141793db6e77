/*
 * cskv.h -- C ABI of the MI355X (gfx950) CSA2 FP4 sparse-decode library.
 *
 * One decode step of CSA2-style compressed sparse attention over an FP4
 * (E2M1) group-quantised KV cache:
 *   1. append: every 2 tokens are compressed into 1 cache entry, quantised to
 *      packed E2M1 codes with one fp32 scale per channel group
 *      (cskv_kv_append_fp4), and the sliding-window rows are written
 *      (cskv_swa_append);
 *   2. the indexer scores every cached entry and keeps the exact top-k
 *      (cskv_indexer_topk);
 *   3-4. the selected entries are gathered, dequantised, and attended to by
 *      all query heads together with the window rows in one softmax
 *      (cskv_sparse_attn_decode);
 *   and the Full / Reindex / Reuse layer modes of one layer group over a
 *   shared cache (cskv_layer_group_decode), optionally with the hierarchical
 *   indexer's candidate pool (cskv_indexer_topk_pool,
 *   cskv_indexer_topk_in_pool, cskv_layer_group_decode_pooled).
 *
 * Sources cited as [P1]/[P2]/[P3] (page title, then the section):
 *   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
 *   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
 *   P3  "KV Cache 瘦身 437 倍：DeepSeek V4.1-Flash 的推理效率革命"
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer and the stream; the library never allocates device memory
 *     and never synchronises.  All work is enqueued on `stream` in order.
 *   - Return value: CSKV_OK (0) or a negative error code.  Arguments are
 *     checked on the host before anything is enqueued; on error nothing is
 *     enqueued and cskv_last_error() (thread-local) describes the problem.
 *   - Conditions only the device can see (capacity overflow, an entries-mode
 *     append onto a pending odd token) set bits in cache->status, which the
 *     caller reads after synchronising; the offending sequence is left
 *     unchanged and no byte outside the cache planes is written.
 *   - Base pointers must be 16-byte aligned.
 */
#ifndef CSKV_H
#define CSKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSKV_OK 0
#define CSKV_EINVAL (-1)        /* bad argument, null pointer, misalignment   */
#define CSKV_EUNSUPPORTED (-2)  /* valid but outside the shapes built here     */
#define CSKV_EWORKSPACE (-3)    /* workspace missing or too small              */
#define CSKV_EHIP (-4)          /* a HIP launch or runtime call failed         */

/* bits of *cache->status (device int32) */
#define CSKV_STATUS_OVERFLOW 1           /* an append would pass capacity       */
#define CSKV_STATUS_ODD_ENTRY_APPEND 2   /* entries-mode append with a pending token */
#define CSKV_STATUS_BAD_STATE 4          /* negative n_tokens or cu_new inconsistent with total_new */
#define CSKV_STATUS_BAD_PAGE 8           /* an append met a block-table entry outside [0, n_pages) */

/*
 * The shared cache of one layer group (device planes, caller-owned).
 *
 * Entry i of sequence b holds the compressed pair of tokens (2i, 2i+1)
 * [P2 三、"突破四：滑动窗口和稀疏注意力" (2 tokens -> 1 entry)]; its 576 numbers
 * are one MLA latent (512) plus its RoPE part (64), shared by all query
 * heads [P2 三、"突破二：MLA，低秩压缩"].  It is stored as E2M1 codes with one
 * fp32 scale per group of channels [P1 §3.1, §4.3; P2 四、"P4 main KV"]:
 *   k_codes  u8  [batch][capacity][dim/2]          two codes per byte, low nibble first
 *   k_scales f32 [batch][capacity][dim/k_group]    scale = group absmax / 6
 * Keys finer, values coarser [P1 §3.1, §4.3]: with v_group > 0 a second plane
 * quantises the value dims (the first dim-rope_dim) with its own group:
 *   v_codes  u8  [batch][capacity][(dim-rope_dim)/2]
 *   v_scales f32 [batch][capacity][(dim-rope_dim)/v_group]
 * otherwise values are read from the key plane (v_codes/v_scales NULL).
 * The indexer key of each entry [P2 四、"CSA2：三种模式"] is kept in bf16
 * (idx_format CSKV_IDX_BF16):
 *   idx_keys bf16 [batch][capacity][idx_dim]
 * or in the pages' FP4 form (idx_format CSKV_IDX_FP4) [P2 四、"890 字节是怎么
 * 算出来的" (a 128-dim indexer key in FP4 is 72 B); P2 四、"P4 main KV" (E2M1
 * with one 8-bit scale per 16 channels, OCP MXFP4)]: E2M1 codes and one E8M0
 * scale byte (the power of two 2^(byte-127)) per 16 dims,
 *   idx_keys   u8 [batch][capacity][idx_dim/2]   (the pointer reinterpreted)
 *   idx_scales u8 [batch][capacity][idx_dim/16]
 * scale = 2^(floor(log2 amax) - 2) of the group's bf16 inputs (byte 0 and
 * zero codes for an all-zero group), codes = nearest E2M1 of x / scale,
 * ties to even, saturating at 6.  Appends take bf16 indexer rows in both
 * formats; scores use the dequantised keys.
 * Sequence state:
 *   n_tokens i32 [batch]  tokens appended so far; entries = n_tokens / 2
 *   pending  f32 [batch][dim]  the odd token waiting for its pair
 *   status   i32 [1]      CSKV_STATUS_* bits, sticky until the caller clears them
 * Supported here: dim 576, rope_dim 64, k_group 32 or 64, v_group 0, 32, 64
 * or 128 (CSKV_KV_MX16: k_group 16, v_group 0 or 16), idx_dim 64 or 128,
 * capacity <= 2^26.
 *
 * Paged planes [P2 三、"突破六：系统层，不改模型改部署" (KV allocated in fixed-
 * size pages, as PagedAttention does, so ragged sequences share one pool)]:
 * with page_size > 0 every entry plane (k/v codes and scales, indexer keys
 * and scales) is [n_pages][page_size][row] instead of [batch][capacity][row],
 * and entry e of sequence b lives in row
 *   block_table[b][e / page_size] * page_size + e % page_size
 * of every plane.  page_size is a power of two, at least 64;
 * capacity = max_pages * page_size (the logical entries per sequence);
 * block_table is device i32 [batch][max_pages]; each plane must stay under
 * 2 GiB.  The table must name a page in [0, n_pages) for every page an
 * append writes or a read covers (entries below n_tokens / ratio); an append
 * that meets any other value writes nothing for that entry and sets
 * CSKV_STATUS_BAD_PAGE; a read through one is no error (the indexer scores
 * the entry from page 0's rows, attention leaves the entry out).  The
 * caller owns the table and may share pages between sequences only for
 * entries that no append writes.  page_size 0: the dense layout above
 * (max_pages, n_pages and block_table unused).
 */
#define CSKV_IDX_BF16 0
#define CSKV_IDX_FP4 1
/* Window rings used with a cache (cskv_sparse_attn_decode, the layer group):
 * bf16 rows, or the pages' FP8 rows [P2 四、"P4 main KV" (the window is kept in
 * FP8)]: OCP E4M3 bytes [batch][window][dim] (the uint16_t pointers of the
 * entry points reinterpreted), written as the nearest E4M3 value, ties to
 * the even mantissa, saturating at +-448, sign kept. */
#define CSKV_SWA_BF16 0
#define CSKV_SWA_FP8 1
/* Scale form of the key and value planes: one fp32 scale = absmax/6 per
 * k_group / v_group channels (CSKV_KV_F32), or the pages' form
 * (CSKV_KV_MX16) [P2 四、"P4 main KV" (E2M1 with one 8-bit scale per 16
 * channels, OCP MXFP4)]: one E8M0 byte per 16 channels, scale =
 * 2^(floor(log2 amax) - 2), codes = nearest E2M1 of x / scale; then k_group
 * is 16, v_group 0 or 16, and k_scales / v_scales are byte planes
 * [batch][capacity][dim/16] / [batch][capacity][(dim-rope_dim)/16]. */
#define CSKV_KV_F32 0
#define CSKV_KV_MX16 1
typedef struct cskv_cache {
    int32_t batch, capacity, dim, rope_dim, k_group, v_group, idx_dim;
    uint8_t *k_codes;
    float *k_scales;
    uint8_t *v_codes;
    float *v_scales;
    uint16_t *idx_keys;
    int32_t *n_tokens;
    float *pending;
    int32_t *status;
    int32_t idx_format;      /* CSKV_IDX_BF16 or CSKV_IDX_FP4 */
    uint8_t *idx_scales;     /* CSKV_IDX_FP4 only, else NULL */
    int32_t swa_format;      /* CSKV_SWA_BF16 or CSKV_SWA_FP8 */
    int32_t k_format;        /* CSKV_KV_F32 or CSKV_KV_MX16 */
    int32_t ratio;           /* tokens per entry: 2 (token pairs compressed into one
                                entry) or 1 (one entry per token, as the decoder cache
                                fed by cskv_ced_project); entries = n_tokens / ratio */
    int32_t page_size;       /* entries per page (a power of two >= 64), or 0: dense planes */
    int32_t max_pages;       /* paged: block-table columns per sequence */
    int32_t n_pages;         /* paged: pages in every plane */
    const int32_t *block_table;  /* paged: device i32 [batch][max_pages] */
} cskv_cache;

/*
 * Append new rows to every sequence of the cache [P2 三、"突破四" (every 2
 * tokens compressed into 1 entry); P1 §3.1 (group FP4 with one scale per
 * group); P1 §3.2 (a trained compressor maps tokens to the compressed form)].
 *
 * tokens   f32 [total_new][dim]; sequence b owns rows cu_new[b]..cu_new[b+1]-1.
 * cu_new   i32 [batch+1] prefix sums, or NULL: one row per sequence
 *          (total_new must equal batch).
 * w_comp   f32 [dim][2*dim] stand-in compressor, or NULL.
 *   non-NULL: rows are tokens.  Tokens pair by absolute position (2i, 2i+1);
 *     the entry is e[r] = sum_j w_comp[r][j] * u[j] with u = x_2i || x_2i+1,
 *     in this fixed fp32 order: the 1152 terms form 64 contiguous blocks of
 *     18, each folded from +0 upward with one fused multiply-add per term,
 *     and the 64 block sums are added as a pairwise tree (blocks 2i and 2i+1
 *     first, then adjacent pairs of those, up to one sum).
 *     A trailing odd token waits in pending[b].  Entry i takes the indexer-key
 *     row of token 2i+1 (the row that completes it); other key rows are unused.
 *   NULL: rows are already entries; each adds 2 tokens.  Requires an even
 *     n_tokens (else CSKV_STATUS_ODD_ENTRY_APPEND, sequence untouched).
 * idx_rows bf16 [total_new][idx_dim] indexer-key rows.
 * Quantisation per group of g channels: a = max|e|, s = a/6 (IEEE fp32
 * division), code = E2M1 of e/s (IEEE division) rounded to nearest with ties
 * to the even code, saturating at 6, sign = sign of e; s == 0 stores scale +0
 * and zero codes.
 * A sequence whose entries would pass capacity is left untouched and sets
 * CSKV_STATUS_OVERFLOW.
 * ws       device workspace for the compressor's fp32 output when w_comp is
 *          non-NULL: at least cskv_append_workspace_bytes(total_new, w_comp)
 *          bytes, 256-byte aligned; ignored (may be NULL) when w_comp is NULL.
 */
int cskv_kv_append_fp4(const cskv_cache *cache, const float *tokens, const int32_t *cu_new,
                       int32_t total_new, const float *w_comp, const uint16_t *idx_rows,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * cskv_kv_append_fp4 with the compressor on the matrix cores for large
 * appends [P1 §3.2 (the compressor is a learned projection: for a prefill
 * chunk, one product of the chunk's token pairs with W)].  Arguments,
 * workspace, quantisation, pending tokens and status are those of
 * cskv_kv_append_fp4, and so is the result of every append that the
 * compressor-free or small-append paths serve (w_comp NULL, cu_new NULL, or
 * fewer than 512 rows).  For an append of 512 rows or more with w_comp, the
 * entry e[r] = sum_j w_comp[r][j] * u[j] is computed with every fp32 factor
 * split into bf16 high and low parts, each term as hi*hi + hi*lo + lo*hi
 * with fp32 accumulation in an unspecified order, so that
 *   |e[r] - sum_j w_comp[r][j] u[j]| <= 2.53e-4 * sum_j |w_comp[r][j] u[j]|
 * (instead of the fixed order of cskv_kv_append_fp4); the codes and scales
 * are then exactly the quantisation of that e.  The fp32 entry rows are left
 * in ws (row r of the append at float offset r * dim) for rows that
 * complete an entry.
 */
int cskv_kv_append_fp4_mfma(const cskv_cache *cache, const float *tokens, const int32_t *cu_new,
                            int32_t total_new, const float *w_comp, const uint16_t *idx_rows,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of cskv_kv_append_fp4 and cskv_kv_append_fp4_mfma: with a
 * compressor, the fp32 compressor rows (total_new * dim * 4), then one
 * 16-byte record per row for the list of rows that complete an entry (used
 * by appends of 512 rows or more) and a count, each region rounded up to 256
 * bytes, and for appends of 512 rows or more the compressor weight split
 * into bf16 high and low parts for the matrix cores (dim * 2*dim * 4 bytes);
 * else a nominal 256. */
size_t cskv_append_workspace_bytes(int32_t total_new, const float *w_comp);

/*
 * Write sliding-window rows [P2 三、"突破四" (each token sees the latest 128);
 * P2 四、"CSA2：三种模式" (every layer keeps its own window)].
 * ring     bf16 [batch][window][dim] (this layer's window, caller-owned)
 * rows     f32 [total_new][dim], grouped by cu_new as in cskv_kv_append_fp4
 *          (cu_new NULL: one row per sequence)
 * end_pos  i32 [batch] token count of each sequence after these rows (e.g.
 *          cache->n_tokens after the append).  The row at absolute position
 *          pos goes to slot pos % window, as bf16 rounded to nearest even, if
 *          it is among the last `window` positions; older rows are skipped.
 */
int cskv_swa_append(uint16_t *ring, int32_t batch, int32_t window, int32_t dim,
                    const float *rows, const int32_t *cu_new, int32_t total_new,
                    const int32_t *end_pos, hipStream_t stream);
/* cskv_swa_append into an FP8 ring (CSKV_SWA_FP8): ring u8 [batch][window][dim]. */
int cskv_swa_append_fp8(uint8_t *ring, int32_t batch, int32_t window, int32_t dim, const float *rows,
                        const int32_t *cu_new, int32_t total_new, const int32_t *end_pos,
                        hipStream_t stream);

/*
 * Indexer scoring and exact top-k [P2 三、"突破四" (a light indexer scores all
 * history and attention keeps the 512 best); P2 四、"CSA2：三种模式" (per-layer
 * indexer query, per-entry indexer key)].
 * Sequence b scores entries j < min(n_tokens[b]/2, capacity):
 *   s_j = sum_h w_h * max(0, sum_d q[b][h][d] * idx_keys[b][j][d])
 * (fp32 accumulation; integer-valued bf16 inputs with |s| < 2^24 are exact).
 * q_idx    bf16 [batch][n_idx_heads][idx_dim], 1 <= n_idx_heads <= 64
 * head_w   f32 [batch][n_idx_heads] or NULL (all weights 1)
 * out_idx  i32 [batch][k]: the k highest scores, ties to the lower index,
 *          listed in ascending index order; -1 pads when fewer than k entries.
 * out_scores f32 [batch][capacity] or NULL (not written): the score s_j of
 *          every entry j < entries of each sequence (a zero score is +0);
 *          rows at and past a sequence's entry count are left untouched.
 * 1 <= k <= 2048.  ws: device workspace of at least
 * cskv_workspace_bytes(cache, CSKV_OP_INDEXER_TOPK, 0, k, 0) bytes, 256-byte
 * aligned (contents need not be initialised; they are overwritten).
 */
int cskv_indexer_topk(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                      const float *head_w, int32_t k, int32_t *out_idx, float *out_scores, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/*
 * Sparse + window attention of one decode step [P2 三、"突破四" (sparse global
 * branch of 512 selected entries plus a 128-token window); P2 三、"突破二"
 * (all heads share one latent entry); P2 四、"P4 main KV" (FP4 is only
 * storage: entries are dequantised before attention)].
 * For every head h of sequence b, one softmax over the keys
 *   { dequantised entry idx[b][t] : 0 <= idx < entries } U { window slot s < swa_len[b] }
 * with logits softmax_scale * q.k over all dim dims; out = sum p * v where
 * v = the value plane (if present) or the first dim-rope_dim key dims;
 * lse = natural log of sum exp(logit).  No keys: out = 0, lse = -inf.
 * q        f32 [batch][n_heads][dim], n_heads a multiple of 16 in [16, 1024]
 * idx      i32 [batch][k], 1 <= k <= 2048 (entries outside [0, entries) are skipped)
 * swa      bf16 [batch][window][dim], 1 <= window <= 1024
 * swa_len  i32 [batch] valid window slots, or NULL: min(n_tokens, window)
 * out      f32 [batch][n_heads][dim-rope_dim];  lse f32 [batch][n_heads] or NULL
 * ws       device workspace for partial softmaxes: at least
 *          cskv_workspace_bytes(cache, CSKV_OP_SPARSE_ATTN, n_heads, k, window)
 *          bytes, 256-byte aligned (may be NULL when that size is 256 or less).
 * The gather addresses a sequence's rows with 32-bit byte offsets, so the
 * cache capacity is limited to 2^23 entries per sequence (CSKV_EUNSUPPORTED).
 */
int cskv_sparse_attn_decode(const cskv_cache *cache, const float *q, int32_t n_heads,
                            const int32_t *idx, int32_t k, const uint16_t *swa, int32_t window,
                            const int32_t *swa_len, float softmax_scale, float *out, float *lse,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Layer modes [P2 四、"CSA2：三种模式，40 层只存 4 份"]. */
#define CSKV_MODE_FULL 0     /* append, own indexer query, own top-k, attend        */
#define CSKV_MODE_REINDEX 1  /* own indexer query over the shared indexer keys      */
#define CSKV_MODE_REUSE 2    /* borrow the most recent FULL/REINDEX index list      */

/* One layer of a group.  Every mode keeps its own query and its own window. */
typedef struct cskv_layer {
    int32_t mode;
    const float *q;          /* f32 [batch][n_heads][dim]                        */
    const uint16_t *q_idx;   /* bf16 [batch][n_idx_heads][idx_dim] (FULL/REINDEX) */
    const float *head_w;     /* f32 [batch][n_idx_heads] or NULL                 */
    uint16_t *swa;           /* bf16 [batch][window][dim] this layer's ring      */
    const float *swa_row;    /* f32 [batch][dim] window row of the new token, or NULL */
    int32_t *idx;            /* i32 [batch][k] written by FULL/REINDEX; unused by REUSE */
    float *out;              /* f32 [batch][n_heads][dim-rope_dim]               */
    float *lse;              /* f32 [batch][n_heads] or NULL                     */
} cskv_layer;

/*
 * One decode step of a CSA2 layer group over its shared cache, layers in
 * order, one new token per sequence [P2 四、"CSA2：三种模式"].
 * new_tokens f32 [batch][dim] and new_idx_rows bf16 [batch][idx_dim] are
 * appended by the first FULL layer (new_tokens NULL: no append).  Every layer
 * with a swa_row writes it at position n_tokens-1 of its own ring.  A REUSE
 * layer needs a FULL or REINDEX layer before it.  ws as for cskv_indexer_topk.
 * layers is a host array.
 */
int cskv_layer_group_decode(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                            const float *new_tokens, const float *w_comp,
                            const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                            int32_t k, int32_t window, float softmax_scale, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * cskv_layer_group_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step with the same results, its workspace taken from
 * a scratch array built into the library (one per GPU, CSKV_NOALLOC_SCRATCH_BYTES
 * bytes, held until the process ends; its address is looked up on the first
 * call on each device).  Nothing is allocated.  A step whose workspace
 * (cskv_workspace_bytes(cache, CSKV_OP_LAYER_GROUP, n_heads, k, window)) is
 * larger returns CSKV_EWORKSPACE before anything is enqueued.  Every call on
 * one GPU shares that GPU's scratch: calls that may overlap on one GPU
 * (different streams, different threads) race and must be serialised by the
 * caller.  The scratch needs no initialisation; the step overwrites what it
 * reads.  Arguments as for cskv_layer_group_decode.
 */
#define CSKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int cskv_layer_group_decode_noalloc(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                                    const float *new_tokens, const float *w_comp,
                                    const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                                    int32_t k, int32_t window, float softmax_scale, hipStream_t stream);

/*
 * Hierarchical sparse indexer [P2 "层级稀疏索引器：后面的层只在候选池里找":
 * after the first Full layer has scored every position, each block of 8
 * positions keeps its best score and the 2048 best blocks, 16,384 positions,
 * form a candidate pool; later Reindex layers score only inside it].
 * Positions are the cache entries; block i holds entries [block*i,
 * block*i + block) below the sequence's entry count.
 *
 * cskv_indexer_topk_pool: cskv_indexer_topk, and from the same scores the
 * pool: the pool_blocks best blocks by their best score (ties: lower block
 * index), ascending block indices in out_pool [batch][pool_blocks], -1
 * padded (fewer blocks than pool_blocks: all of them).
 * cskv_indexer_topk_in_pool: the exact top-k of a layer's own indexer scores
 * restricted to the entries of the pooled blocks (ties: lower entry index),
 * ascending, -1 padded; pool as written by cskv_indexer_topk_pool on the
 * same cache state.
 * pool_block in {2, 4, 8, 16}; 1 <= pool_blocks <= 2048 and
 * pool_blocks * pool_block >= k + pool_block (so a pool of more than k
 * entries exists whenever the sequence has more than k).  Other arguments as
 * for cskv_indexer_topk.  ws: cskv_workspace_bytes_pool(cache,
 * CSKV_OP_INDEXER_POOL or CSKV_OP_INDEXER_IN_POOL, 0, k, 0, pool_blocks,
 * pool_block) bytes, 256-byte aligned.
 */
int cskv_indexer_topk_pool(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                           const float *head_w, int32_t k, int32_t *out_idx, int32_t pool_blocks,
                           int32_t pool_block, int32_t *out_pool, void *ws, size_t ws_bytes,
                           hipStream_t stream);
int cskv_indexer_topk_in_pool(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                              const float *head_w, int32_t k, const int32_t *pool, int32_t pool_blocks,
                              int32_t pool_block, int32_t *out_idx, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * cskv_layer_group_decode with the hierarchical indexer: the first FULL
 * layer also builds the candidate pool (pool_blocks blocks of pool_block
 * entries), and every REINDEX layer after it selects inside the pool
 * (cskv_indexer_topk_in_pool); a REINDEX layer before any FULL layer scans
 * every entry.  pool_blocks = 0 is cskv_layer_group_decode.  ws:
 * cskv_workspace_bytes_pool(cache, CSKV_OP_LAYER_GROUP, n_heads, k, window,
 * pool_blocks, pool_block) bytes; the pool itself lives in it.
 */
int cskv_layer_group_decode_pooled(const cskv_cache *cache, const cskv_layer *layers,
                                   int32_t n_layers, const float *new_tokens, const float *w_comp,
                                   const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                                   int32_t k, int32_t window, float softmax_scale, int32_t pool_blocks,
                                   int32_t pool_block, void *ws, size_t ws_bytes, hipStream_t stream);

/* Device workspace bytes an operation needs (at least 256); 0 on invalid
 * arguments (see cskv_last_error).  op: CSKV_OP_INDEXER_TOPK (uses k),
 * CSKV_OP_SPARSE_ATTN (n_heads, k, window), CSKV_OP_LAYER_GROUP (all).
 * cskv_workspace_bytes_pool also takes the pool's size, for
 * CSKV_OP_INDEXER_POOL, CSKV_OP_INDEXER_IN_POOL (k and the pool) and
 * CSKV_OP_LAYER_GROUP (all; pool_blocks = 0: no pool). */
#define CSKV_OP_INDEXER_TOPK 1
#define CSKV_OP_SPARSE_ATTN 2
#define CSKV_OP_LAYER_GROUP 3
#define CSKV_OP_INDEXER_POOL 4
#define CSKV_OP_INDEXER_IN_POOL 5
size_t cskv_workspace_bytes(const cskv_cache *cache, int32_t op, int32_t n_heads, int32_t k,
                            int32_t window);
size_t cskv_workspace_bytes_pool(const cskv_cache *cache, int32_t op, int32_t n_heads, int32_t k,
                                 int32_t window, int32_t pool_blocks, int32_t pool_block);

/*
 * The CED projection [P2 四、"CED：上半段模型的 KV 由下半段代算" (the second
 * half's global KV is the first half's last output times a per-layer
 * projection)]: out[r][n] = sum_k h[r][k] * w[n][k] for r < rows, n < n_out.
 *
 * h     bf16 [rows][d_model] (device), the hidden states
 * w     bf16 [n_out][d_model] (device), one row per output channel
 * out   f32 [rows][n_out] (device), written; it may not overlap h or w
 * d_model a multiple of 128 in [128, 65536]; n_out a multiple of 16; rows in
 * [0, 2^22]; all pointers 16-byte aligned.  bf16 MFMA with fp32
 * accumulation: each output is the sum of its products in a fixed order
 * (exact whenever the inputs make every partial sum representable, e.g.
 * small integers times a common power of two).  Enqueued on `stream`.
 */
int cskv_ced_project(const uint16_t *h, int64_t rows, int32_t d_model, const uint16_t *w, int32_t n_out,
                     float *out, hipStream_t stream);

/*
 * One group of the layer plan: the layers that share one cache and the
 * source of the step's new entry per sequence [P2 四、"CSA2：三种模式，40 层只存
 * 4 份" (encoder groups of Full + 5 Reuse with 2->1 caches; the decoder's
 * groups, Full + 3 Reuse and then Reindex + 3 Reuse, read one cache);
 * "CED：上半段模型的 KV 由下半段代算"].
 *
 * new_tokens + w_comp: one new token per sequence through the 2->1
 *   compressor (ratio-2 cache), as cskv_layer_group_decode; w_comp NULL:
 *   new_tokens are entries.
 * ced_h + ced_w + d_model: the new entry of each sequence is the CED
 *   projection of ced_h (bf16 [batch][d_model]) by ced_w (bf16
 *   [dim][d_model]), appended as an entry (one per token on a ratio-1 cache).
 * Neither: no append.  new_idx_rows bf16 [batch][idx_dim] goes with either.
 * pool_blocks, pool_block: the hierarchical indexer for this group's REINDEX
 *   layers (0, 0: off).  layers: host array as for cskv_layer_group_decode.
 */
typedef struct cskv_group {
    const cskv_cache *cache;
    const cskv_layer *layers;
    int32_t n_layers;
    const float *new_tokens;
    const float *w_comp;
    const uint16_t *ced_h;
    const uint16_t *ced_w;
    int32_t d_model;
    const uint16_t *new_idx_rows;
    int32_t pool_blocks, pool_block;
} cskv_group;

/*
 * One decode step of every group in order, each as cskv_layer_group_decode
 * (cskv_layer_group_decode_pooled when its pool is set), after the CED
 * projection for a group that has one.  Every group is checked before
 * anything is enqueued; an error leaves every cache untouched.  groups is a
 * host array of 1..64 groups sharing n_idx_heads, n_heads, k and window.
 * ws: cskv_model_workspace_bytes bytes, 256-byte aligned, reused by the
 * groups in turn.  Returns CSKV_OK or an error code.
 */
int cskv_model_decode(const cskv_group *groups, int32_t n_groups, int32_t n_idx_heads, int32_t n_heads,
                      int32_t k, int32_t window, float softmax_scale, void *ws, size_t ws_bytes,
                      hipStream_t stream);
size_t cskv_model_workspace_bytes(const cskv_group *groups, int32_t n_groups, int32_t n_heads, int32_t k,
                                  int32_t window);

/* Bytes one entry occupies across all planes (codes, scales, indexer key)
 * [P2 四、"890 字节是怎么算出来的"]. */
size_t cskv_entry_bytes(int32_t dim, int32_t rope_dim, int32_t k_group, int32_t v_group,
                        int32_t idx_dim);

/* Bytes one entry of *cache occupies in the cache's own formats
 * [P2 四、"P4 main KV" and "890 字节是怎么算出来的"]: key codes dim/2, key
 * scales 4 B per k_group channels (CSKV_KV_F32) or 1 B per 16 (CSKV_KV_MX16),
 * the value plane likewise when v_group > 0, and the indexer key: 2 B per
 * dim (CSKV_IDX_BF16) or idx_dim/2 + idx_dim/16 (CSKV_IDX_FP4).  In the
 * pages' formats with split planes the value row (512 latent dims) is 288 B
 * and the indexer key 72 B.  Host only; the plane pointers are checked for
 * presence and alignment but never read.  Returns 0 for a descriptor that
 * every entry point would reject (cskv_last_error says why). */
size_t cskv_cache_entry_bytes(const cskv_cache *cache);

/* Thread-local description of the last error (host string, never NULL). */
const char *cskv_last_error(void);

/*
 * Kernel timers for measurement.  When enabled for a kernel kind, each of
 * the next `max_launches` launch groups of that kind (the one to three
 * kernels one call launches for it) records an event as its first kernel
 * starts and one as its last kernel ends, passed to hipExtLaunchKernel, so no
 * marker packets are added to the stream.  cskv_timer_read waits for them
 * and returns the summed milliseconds and the count.  cskv_timer_pause(kind,
 * 1) stops recording for that kind (launches run untimed) until
 * cskv_timer_pause(kind, 0), so a bench can time a sample of its steps.  Not
 * thread-safe; meant for benches.  CSKV_KERNEL_COMPRESS times the stand-in
 * compressor's kernel of an append alone; when it and CSKV_KERNEL_APPEND are
 * both on, the APPEND interval then starts at the quantiser (the kernel
 * after the compressor).
 */
#define CSKV_KERNEL_APPEND 1
#define CSKV_KERNEL_SWA_APPEND 2
#define CSKV_KERNEL_INDEXER_SCAN 3
#define CSKV_KERNEL_TOPK_SELECT 4
#define CSKV_KERNEL_ATTENTION 5
#define CSKV_KERNEL_COMPRESS 6
int cskv_timer_enable(int32_t kernel_kind, int32_t max_launches);
int cskv_timer_pause(int32_t kernel_kind, int32_t paused);
int cskv_timer_read(int32_t kernel_kind, double *total_ms, int32_t *count);
int cskv_timer_disable_all(void);

#ifdef __cplusplus
}
#endif
#endif
