/*
 * cskv_oracle.h -- plain CPU oracle of the CSA2 FP4 sparse-decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the HIP library is checked against.  Only the test suite,
 * the smoke check and the bench's CPU-baseline leg may load it; the product
 * path never links, loads or calls it, and it shares no code with the HIP
 * sources.
 *
 * Arithmetic: fp64 for every floating-point result that has a plain
 * mathematical definition (indexer scores, attention); fp32 where the method
 * is an encoding whose decisions are defined in fp32 (group scale, the
 * division by it, the stand-in compressor's fused multiply-add chain).
 *
 * Sources cited as [P1]/[P2]/[P3] (page title, then the section):
 *   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
 *   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
 *   P3  "KV Cache 瘦身 437 倍：DeepSeek V4.1-Flash 的推理效率革命"
 *
 * Parity status per function is stated at each declaration.
 */
#ifndef CSKV_ORACLE_H
#define CSKV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------- byte accounting ---------------------------------------- */

/* KV bytes = 2 x layers x tokens x heads x head_dim x bytes per element; the 2
 * counts K and V [P1 §1; P2 "KV Cache 到底有多大"].
 * Pinned: the pages' own worked numbers (95-layer BF16 model per token; the
 * L=60 H=64 D=128 64K FP16 estimate; 128K / 1M context sizes). */
uint64_t orc_kv_bytes(uint64_t layers, uint64_t tokens, uint64_t heads,
                      uint64_t head_dim, uint64_t elem_bytes);

/* Bytes of one group-quantised FP4 row: dims/2 code bytes + one scale of
 * scale_bytes per group [P1 §3.1; P2 "890 字节是怎么算出来的"].
 * Pinned: 512-dim main entry with 16-channel 1-byte scales = 288 B; 128-dim
 * indexer key = 72 B (both printed on P2). */
double orc_fp4_row_bytes(int dims, int group, double scale_bytes);

/* Per-token global KV of a CSA2 model: sum over cache copies of
 * (main entry + indexer key bytes) / compression ratio
 * [P2 "890 字节是怎么算出来的", "CSA2：三种模式，40 层只存 4 份"].
 * Pinned: 3 encoder copies at ratio 2 + 1 decoder copy at ratio 1 = 900 B. */
double orc_global_kv_per_token(int n_copies, const int *ratio,
                               double main_entry_bytes, double idx_entry_bytes);

/* ---------------- E2M1 (FP4) and bf16 ------------------------------------ */

/* Value of a 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit
 * [P1 §3.1; P2 "P4 main KV"].  Pinned: the 16 codes give exactly
 * {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}. */
double orc_e2m1_value(unsigned code);

/* Nearest E2M1 code to v (compared in fp64), ties to the even code, values
 * past 6 saturate to 6, sign bit = signbit(v).  v must be finite.
 * Pinned: exhaustive comparison over all fp32 inputs with the midpoint table
 * (tests/native), plus round-trip and monotonicity. */
unsigned orc_e2m1_encode(float v);

/* Nearest bf16 to x, ties to even mantissa; overflow past the largest finite
 * bf16 (by more than half an ulp) gives infinity.  x must be finite.
 * Pinned: exhaustive comparison with the integer round-half-even trick. */
uint16_t orc_bf16_from_f32(float x);
double orc_bf16_value(uint16_t h);

/* ---------------- compress, quantise, append ----------------------------- */

/* Stand-in for the learned 2->1 compressor [P2 "突破四"; P1 §3.2]:
 * e[r] = sum_j W[r][j] * u[j], u = x_even || x_odd, in a fixed fp32 order:
 * the 2D terms are cut into 64 contiguous blocks of 2D/64; each block is
 * folded from its first term upward with one fused multiply-add per term,
 * starting from +0; the 64 block sums are then added as a pairwise tree
 * (blocks 2i and 2i+1, then adjacent pairs of those, and so on).
 * The pages' compressor is trained and not given: parity with it is
 * unpinned.  The order is pinned by cases that round differently under
 * other groupings, and the result against an fp64 evaluation within the
 * forward-error bound of this order (2D/64 + 6 roundings per term). */
void orc_compress_pair(const float *W, const float *x_even, const float *x_odd,
                       int dim, float *e);

/* Group FP4 quantisation of one row [P1 §3.1, §4.3; P2 "P4 main KV"]:
 * per contiguous group of `group` channels, a = max|x|, s = a/6 (fp32 IEEE
 * division), codes = E2M1(x/s) with x/s an fp32 IEEE division; s == 0 stores
 * scale +0 and all-zero codes.  Two codes per byte, low nibble first.
 * Pinned: decode error bound, "every non-zero group holds a +-6 code",
 * zero groups, sign of tiny negatives, exact round trip. */
void orc_quantize_row(const float *x, int n, int group, uint8_t *packed, float *scales);
void orc_dequantize_row(const uint8_t *packed, const float *scales, int n, int group,
                        double *out);

/* Host mirror of the device cache (same layout as the HIP library's). */
typedef struct {
    int32_t batch, capacity, dim, rope_dim, k_group, v_group, idx_dim;
    uint8_t *k_codes;   /* [B][cap][dim/2]                 */
    float *k_scales;    /* [B][cap][dim/k_group]           */
    uint8_t *v_codes;   /* [B][cap][(dim-rope)/2] or NULL  */
    float *v_scales;    /* [B][cap][(dim-rope)/v_group]    */
    uint16_t *idx_keys; /* [B][cap][idx_dim] bf16 (format 0) or E2M1 codes,
                           idx_dim/2 bytes per row (format 1) */
    int32_t *n_tokens;  /* [B] tokens seen                 */
    float *pending;     /* [B][dim] odd token awaiting its pair */
    int32_t *status;    /* [1] bit flags                   */
    int32_t idx_format; /* 0: bf16 indexer keys; 1: E2M1 + E8M0 per 16 dims */
    uint8_t *idx_scales;/* [B][cap][idx_dim/16] E8M0 bytes (format 1) */
    int32_t swa_format; /* window rings used with this cache: 0 bf16, 1 FP8 E4M3 */
    int32_t k_format;   /* 0: fp32 scale per k_group/v_group channels; 1: one E8M0 byte
                           per 16 channels in both planes (k_group 16, v_group 0 or 16;
                           k_scales / v_scales reinterpreted as bytes) */
    int32_t ratio;      /* tokens per entry: 2 (token pairs compressed into one entry,
                           the encoder caches) or 1 (one entry per token, the decoder
                           cache fed by the CED projection) [P2 四、"CSA2：三种模式，
                           40 层只存 4 份"; "890 字节是怎么算出来的"] */
} orc_cache;

#define ORC_STATUS_OVERFLOW 1
#define ORC_STATUS_ODD_ENTRY_APPEND 2

/* Append new rows to every sequence (2 tokens -> 1 entry, [P2 "突破四"]).
 * tokens fp32 [total][dim]; cu_new [B+1] prefix sums of rows per sequence.
 * w_comp != NULL: rows are tokens, paired by absolute position (2i, 2i+1);
 *   an odd trailing token waits in pending[b]; entry i takes the indexer-key
 *   row of the token that completes it.  Ratio-2 caches only.
 * w_comp == NULL: rows are already entries (n_tokens += ratio per row); a
 *   ratio-2 cache requires an even token count.
 * A sequence whose entries would pass capacity is left untouched and raises
 * ORC_STATUS_OVERFLOW. */
void orc_kv_append(orc_cache *c, const float *tokens, const int32_t *cu_new,
                   const float *w_comp, const uint16_t *idx_rows);

/* Write the window rows of a step: for each new row of sequence b at absolute
 * position pos (the rows end at end_pos[b]), rows inside the last W positions
 * go to ring slot pos % W as bf16 [P2 "突破四"; "CSA2：三种模式"]. */
void orc_swa_append(uint16_t *ring, int batch, int W, int dim, const float *rows,
                    const int32_t *cu_new, const int32_t *end_pos);

/* ---------------- CED projection ----------------------------------------- */

/* The decoder's global KV from one hidden state [P2 四、"CED：上半段模型的
 * KV 由下半段代算" (the second half's KV is the first half's last output
 * times a per-layer projection)]: out[r][n] = sum_k h[r][k] * w[n][k] over
 * k < d_model, h bf16 [rows][d_model], w bf16 [n_out][d_model] (one row per
 * output channel), summed in fp64 and rounded once to fp32.  Parity: pinned
 * by closed forms (identity and rank-1 weights, linearity) and by exact
 * integer brute force. */
void orc_ced_project(const uint16_t *h, int64_t rows, int d_model, const uint16_t *w, int n_out,
                     float *out);

/* ---------------- FP4 indexer key ---------------------------------------- */

/* The pages' indexer-key format [P2 四、"890 字节是怎么算出来的" (a 128-dim
 * indexer key stored in FP4 takes 72 B); P2 四、"P4 main KV" (E2M1, one 8-bit
 * scale per 16 channels, the OCP MXFP4 family)]: E2M1 codes (low nibble =
 * even dim) and one E8M0 scale per 16 consecutive dims.  E8M0 byte s is the
 * power of two 2^(s-127).  Scale of a group with largest magnitude a > 0:
 * 2^(floor(log2 a) - 2) (the MX rule, 2 being E2M1's largest exponent);
 * a = 0 gives byte 0 and zero codes.  Codes: orc_e2m1_encode(x / scale), the
 * division by a power of two being exact.  Pinned: the E8M0 values, the scale
 * rule at binade edges, exact round trips, the hand-derived mapping of the
 * integers -8..8, and 72 B per 128 dims. */
double orc_e8m0_value(uint8_t s);
void orc_quantize_mx16(const uint16_t *x_bf16, int n, uint8_t *codes, uint8_t *scales);
void orc_dequantize_mx16(const uint8_t *codes, const uint8_t *scales, int n, double *out);
/* The same form for a main-entry plane [P2 四、"P4 main KV" (E2M1, one 8-bit
 * scale per 16 channels, OCP MXFP4)]: fp32 inputs, the MX scale rule on the
 * group's largest fp32 magnitude, codes as above. */
void orc_quantize_mx16_f32(const float *x, int n, uint8_t *codes, uint8_t *scales);

/* ---------------- FP8 window rows ---------------------------------------- */

/* The pages keep the sliding-window rows in FP8 [P2 四、"P4 main KV" (the
 * window is stored in FP8); P2 三、"突破四" (the 128-token window)].  Format:
 * OCP E4M3 -- 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, 0x7F/0xFF NaN, largest finite 448, subnormals k * 2^-9.
 * Encoding: the nearest E4M3 value, ties to the even mantissa, magnitudes
 * past 448 saturate to 448, sign kept (so -0 is 0x80).  Pinned: all 254
 * finite values from their fields, round trips, midpoints, saturation. */
double orc_e4m3_value(uint8_t v);
uint8_t orc_e4m3_encode(float x);
/* orc_swa_append with an FP8 ring */
void orc_swa_append_fp8(uint8_t *ring, int batch, int W, int dim, const float *rows,
                        const int32_t *cu_new, const int32_t *end_pos);

/* ---------------- indexer + top-k ---------------------------------------- */

/* s_j = sum_h w_h * max(0, sum_d q[h][d] K[j][d]) in fp64, over j < E
 * [P2 "突破四" (lightweight indexer scoring all history),
 *  "CSA2：三种模式" (per-layer indexer Q, per-entry indexer K)].
 * The formula is not printed on the pages; parity with the model's indexer
 * is unpinned.  Pinned: exact integer identities and brute-force cases. */
void orc_indexer_scores(const uint16_t *keys, int64_t E, int idx_dim,
                        const uint16_t *q, int heads, const float *head_w,
                        double *scores);

/* Exact top-k: order by (score descending, index ascending), take the first
 * min(k, E), output them ascending by index, pad with -1 [P2 "突破四": keep
 * the 512 highest].  Pinned: brute force over all subsets on tiny inputs,
 * threshold invariants, forced ties. */
void orc_topk(const double *scores, int64_t E, int k, int32_t *out);

/* Whole-batch indexer + top-k on a cache: sequence b scores its first
 * n_tokens[b]/2 entries (capped at capacity) with its stored indexer keys
 * (bf16, or the dequantised FP4 keys of format 1). q [B][H][Di], head_w
 * [B][H] or NULL, out [B][k]. */
void orc_indexer_topk(const orc_cache *c, const uint16_t *q, int heads,
                      const float *head_w, int k, int32_t *out);

/* ---------------- hierarchical indexer: the candidate pool ---------------- */

/* Candidate pool [P2 "层级稀疏索引器：后面的层只在候选池里找": the first Full
 * layer scores every position, each block of 8 positions keeps its highest
 * score, the 2048 best blocks form a 16,384-position pool].  Positions are
 * the E entries; block i holds entries [block*i, block*i + block) that are
 * < E (the last block may be short); its score is the highest score among
 * them.  The pool is the first min(nb, blocks) blocks ordered by (block
 * score descending, block index ascending) -- the top-k tie rule applied to
 * blocks -- output ascending by block index, padded with -1.
 * Pinned: brute force over all block subsets on tiny inputs, hand-built
 * cases, and the closed forms stated in orc_topk_in_pool. */
void orc_pool_blocks(const double *scores, int64_t E, int block, int nb, int32_t *pool);

/* Top-k inside a pool [same passage: later Reindex layers score only inside
 * the pool]: among the entries of the pooled blocks (those < E), order by
 * (score descending, entry index ascending), take the first min(k, count),
 * output ascending by entry index, pad with -1.
 * Pinned: brute force on tiny inputs; when every block is pooled the result
 * is orc_topk's; with the pool's own scores, distinct scores and k <= nb it
 * is orc_topk's as well (each of the k best entries lies in a block whose
 * maximum is among the k best block maxima). */
void orc_topk_in_pool(const double *scores, int64_t E, const int32_t *pool, int nb, int block,
                      int k, int32_t *out);

/* Whole-batch forms on a cache, scores as orc_indexer_scores: pool [B][nb];
 * out [B][k]. */
void orc_indexer_pool(const orc_cache *c, const uint16_t *q, int heads, const float *head_w,
                      int block, int nb, int32_t *pool);
void orc_indexer_topk_in_pool(const orc_cache *c, const uint16_t *q, int heads,
                              const float *head_w, const int32_t *pool, int nb, int block, int k,
                              int32_t *out);

/* ---------------- attention ---------------------------------------------- */

/* One joint softmax per query head over the selected compressed entries and
 * the window rows [P2 "突破四"; "突破二" (one shared latent for all heads)]:
 * l = scale * q.k; out = sum softmax(l) * v[0:dim-rope]; lse = log sum exp l.
 * Keys: K = dequantised key plane (all dim dims); values: the value plane if
 * present, else K's first dim-rope dims.  Indices < 0 or >= the sequence's
 * entry count are skipped.  No keys: out = 0, lse = -inf.
 * q fp32 [B][Hq][dim]; idx [B][k]; swa bf16 [B][W][dim] (FP8 E4M3 bytes when
 * the cache's swa_format is 1, the pointer reinterpreted); swa_len [B]
 * (NULL: min(n_tokens, W)); out [B][Hq][dim-rope]; lse [B][Hq].
 * Pinned: equal logits -> mean of values, a dominant logit -> its value,
 * single key, LSE merge of the two branches, permutation invariance. */
void orc_sparse_attn(const orc_cache *c, const float *q, int heads, const int32_t *idx,
                     int k, const uint16_t *swa, int W, const int32_t *swa_len,
                     double scale, double *out, double *lse);

#ifdef __cplusplus
}
#endif
#endif
