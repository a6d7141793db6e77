/*
 * cskv_oracle.c -- plain CPU oracle of the CSA2 FP4 sparse-decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * bench's CPU-baseline leg, never by the product path.  Shares no code with
 * the HIP library.  Each function follows the passage cited in
 * cskv_oracle.h; the code is written for checking by eye, not for speed.
 * The only parallelism is an OpenMP loop over independent sequences.
 */
#include "cskv_oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ accounting */

uint64_t orc_kv_bytes(uint64_t layers, uint64_t tokens, uint64_t heads,
                      uint64_t head_dim, uint64_t elem_bytes)
{
    return 2u * layers * tokens * heads * head_dim * elem_bytes;
}

double orc_fp4_row_bytes(int dims, int group, double scale_bytes)
{
    return dims * 0.5 + (double)(dims / group) * scale_bytes;
}

double orc_global_kv_per_token(int n_copies, const int *ratio,
                               double main_entry_bytes, double idx_entry_bytes)
{
    double total = 0.0;
    for (int i = 0; i < n_copies; ++i)
        total += (main_entry_bytes + idx_entry_bytes) / ratio[i];
    return total;
}

/* ------------------------------------------------------------ E2M1, bf16 */

double orc_e2m1_value(unsigned code)
{
    unsigned sign = (code >> 3) & 1u, expo = (code >> 1) & 3u, mant = code & 1u;
    double mag;
    if (expo == 0)
        mag = 0.5 * mant;                               /* subnormal: m x 2^(1-bias) x 0.5 */
    else
        mag = ldexp(1.0 + 0.5 * mant, (int)expo - 1);   /* normal: 2^(e-1) x (1 + m/2) */
    return sign ? -mag : mag;
}

unsigned orc_e2m1_encode(float v)
{
    assert(isfinite(v));
    double mag = fabs((double)v);
    unsigned sign = signbit(v) ? 8u : 0u;
    /* at or past the largest grid value the nearest point is 6 (saturation);
       handled first because for huge inputs the fp64 distances to 4 and 6
       round to the same number */
    if (mag >= 6.0) return 7u | sign;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        double d = fabs(mag - orc_e2m1_value(c));
        /* strictly closer wins; on an exact tie the even code wins (the two
           candidates of a tie are neighbours, so exactly one is even) */
        if (d < best_d || (d == best_d && (c & 1u) == 0)) {
            best = c;
            best_d = d;
        }
    }
    /* below 6 every distance is exact in fp64: an fp32 input and a grid value
       of at most 3 significant bits differ by a number of at most ~30 bits */
    return best | sign;
}

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

double orc_bf16_value(uint16_t h)
{
    return (double)bits_f32((uint32_t)h << 16);
}

uint16_t orc_bf16_from_f32(float x)
{
    assert(isfinite(x));
    uint32_t u = f32_bits(x);
    uint16_t lo = (uint16_t)(u >> 16);           /* truncation toward zero */
    uint16_t hi = (uint16_t)(lo + 1);            /* next bf16 away from zero */
    double xd = fabs((double)x);
    double vlo = fabs(orc_bf16_value(lo));
    /* the successor of the largest finite bf16 is infinity; for rounding it
       sits where the next binade would start */
    double vhi = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128) : fabs(orc_bf16_value(hi));
    double dlo = xd - vlo, dhi = vhi - xd;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;                  /* tie: even mantissa */
}

/* ------------------------------------------------------------ compress */

#define ORC_COMPRESS_BLOCKS 64

void orc_compress_pair(const float *W, const float *x_even, const float *x_odd,
                       int dim, float *e)
{
    const int n = 2 * dim;
    assert(n % ORC_COMPRESS_BLOCKS == 0);
    const int per = n / ORC_COMPRESS_BLOCKS;
    for (int r = 0; r < dim; ++r) {
        float part[ORC_COMPRESS_BLOCKS];
        for (int p = 0; p < ORC_COMPRESS_BLOCKS; ++p) {       /* block sums */
            float acc = 0.0f;
            for (int j = p * per; j < (p + 1) * per; ++j) {
                float u = (j < dim) ? x_even[j] : x_odd[j - dim];
                acc = fmaf(W[(size_t)r * n + j], u, acc);
            }
            part[p] = acc;
        }
        for (int w = 1; w < ORC_COMPRESS_BLOCKS; w *= 2)      /* pairwise tree */
            for (int p = 0; p < ORC_COMPRESS_BLOCKS; p += 2 * w)
                part[p] = part[p] + part[p + w];
        e[r] = part[0];
    }
}

/* ------------------------------------------------------------ quantise */

void orc_quantize_row(const float *x, int n, int group, uint8_t *packed, float *scales)
{
    assert(n % group == 0 && n % 2 == 0);
    unsigned *code = (unsigned *)malloc(sizeof(unsigned) * (size_t)n);
    for (int g0 = 0; g0 < n; g0 += group) {
        float a = 0.0f;
        for (int c = g0; c < g0 + group; ++c) {
            assert(isfinite(x[c]));
            a = fmaxf(a, fabsf(x[c]));
        }
        float s = a / 6.0f;
        if (s == 0.0f) {
            scales[g0 / group] = 0.0f;
            for (int c = g0; c < g0 + group; ++c) code[c] = 0;
        } else {
            scales[g0 / group] = s;
            for (int c = g0; c < g0 + group; ++c) code[c] = orc_e2m1_encode(x[c] / s);
        }
    }
    for (int t = 0; t < n / 2; ++t)
        packed[t] = (uint8_t)(code[2 * t] | (code[2 * t + 1] << 4));
    free(code);
}

void orc_dequantize_row(const uint8_t *packed, const float *scales, int n, int group,
                        double *out)
{
    for (int c = 0; c < n; ++c) {
        unsigned code = (c & 1) ? (packed[c / 2] >> 4) : (packed[c / 2] & 0xFu);
        out[c] = orc_e2m1_value(code) * (double)scales[c / group];
    }
}

/* ------------------------------------------------------------ cache append */

/* ------------------------------------------------------------ FP8 window rows */

double orc_e4m3_value(uint8_t v)
{
    const int sign = v >> 7, ex = (v >> 3) & 15, man = v & 7;
    if (ex == 15 && man == 7) return NAN;
    double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

uint8_t orc_e4m3_encode(float x)
{
    assert(isfinite(x));
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double mag = fabs((double)x);
    if (mag >= 448.0) return sign | 0x7E;
    /* the nearest of the 127 non-negative finite values; on a tie the even
       mantissa (the two candidates of a tie are neighbours) */
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 0x7F; ++c) {
        double d = fabs(mag - orc_e4m3_value((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1u) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

void orc_swa_append_fp8(uint8_t *ring, int batch, int W, int dim, const float *rows,
                        const int32_t *cu_new, const int32_t *end_pos)
{
    for (int b = 0; b < batch; ++b) {
        int64_t m = cu_new[b + 1] - cu_new[b];
        for (int64_t q = 0; q < m; ++q) {
            int64_t pos = (int64_t)end_pos[b] - m + q;
            if (pos < 0 || pos < (int64_t)end_pos[b] - W) continue;
            const float *x = rows + (size_t)(cu_new[b] + q) * dim;
            uint8_t *dst = ring + ((size_t)b * W + (size_t)(pos % W)) * dim;
            for (int d = 0; d < dim; ++d) dst[d] = orc_e4m3_encode(x[d]);
        }
    }
}

/* ------------------------------------------------------------ FP4 indexer key */

double orc_e8m0_value(uint8_t s)
{
    return ldexp(1.0, (int)s - 127);
}

void orc_quantize_mx16(const uint16_t *x_bf16, int n, uint8_t *codes, uint8_t *scales)
{
    for (int g = 0; g < n / 16; ++g) {
        double a = 0.0;
        for (int i = 0; i < 16; ++i) {
            double v = fabs(orc_bf16_value(x_bf16[16 * g + i]));
            if (v > a) a = v;
        }
        int e = -127;
        if (a > 0.0) {
            int ex;
            (void)frexp(a, &ex);          /* a = m * 2^ex, 0.5 <= m < 1: floor(log2 a) = ex - 1 */
            e = ex - 1 - 2;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 16; i += 2) {
            unsigned c0 = 0, c1 = 0;
            if (a > 0.0) {
                c0 = orc_e2m1_encode((float)ldexp(orc_bf16_value(x_bf16[16 * g + i]), -e));
                c1 = orc_e2m1_encode((float)ldexp(orc_bf16_value(x_bf16[16 * g + i + 1]), -e));
            }
            codes[(16 * g + i) / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

void orc_quantize_mx16_f32(const float *x, int n, uint8_t *codes, uint8_t *scales)
{
    for (int g = 0; g < n / 16; ++g) {
        double a = 0.0;
        for (int i = 0; i < 16; ++i) {
            double v = fabs((double)x[16 * g + i]);
            if (v > a) a = v;
        }
        int e = -127;
        if (a > 0.0) {
            int ex;
            (void)frexp(a, &ex);          /* floor(log2 a) = ex - 1 */
            e = ex - 1 - 2;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 16; i += 2) {
            unsigned c0 = 0, c1 = 0;
            if (a > 0.0) {
                c0 = orc_e2m1_encode((float)ldexp((double)x[16 * g + i], -e));
                c1 = orc_e2m1_encode((float)ldexp((double)x[16 * g + i + 1], -e));
            }
            codes[(16 * g + i) / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

void orc_dequantize_mx16(const uint8_t *codes, const uint8_t *scales, int n, double *out)
{
    for (int i = 0; i < n; ++i) {
        unsigned c = (codes[i / 2] >> (4 * (i % 2))) & 15u;
        out[i] = orc_e2m1_value(c) * orc_e8m0_value(scales[i / 16]);
    }
}

static void store_entry(orc_cache *c, int b, int64_t i, const float *e, const uint16_t *idx_row)
{
    const int D = c->dim, Dv = c->dim - c->rope_dim;
    size_t row = (size_t)b * c->capacity + (size_t)i;
    if (c->k_format == 1) {
        orc_quantize_mx16_f32(e, D, c->k_codes + row * (D / 2), (uint8_t *)c->k_scales + row * (D / 16));
        if (c->v_group > 0)
            orc_quantize_mx16_f32(e, Dv, c->v_codes + row * (Dv / 2), (uint8_t *)c->v_scales + row * (Dv / 16));
    } else {
        orc_quantize_row(e, D, c->k_group, c->k_codes + row * (D / 2),
                         c->k_scales + row * (D / c->k_group));
        if (c->v_group > 0)
            orc_quantize_row(e, Dv, c->v_group, c->v_codes + row * (Dv / 2),
                             c->v_scales + row * (Dv / c->v_group));
    }
    if (c->idx_format == 1)
        orc_quantize_mx16(idx_row, c->idx_dim, (uint8_t *)c->idx_keys + row * (c->idx_dim / 2),
                          c->idx_scales + row * (c->idx_dim / 16));
    else
        memcpy(c->idx_keys + row * c->idx_dim, idx_row, sizeof(uint16_t) * (size_t)c->idx_dim);
}

static void raise_status(orc_cache *c, int32_t bit)
{
    #pragma omp atomic
    c->status[0] |= bit;
}

void orc_kv_append(orc_cache *c, const float *tokens, const int32_t *cu_new,
                   const float *w_comp, const uint16_t *idx_rows)
{
    const int D = c->dim;
    /* sequences are independent: each touches only its own rows and state */
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < c->batch; ++b) {
        float *e = (float *)malloc(sizeof(float) * (size_t)D);
        int64_t p = c->n_tokens[b];
        int64_t m = cu_new[b + 1] - cu_new[b];
        const float *rows = tokens + (size_t)cu_new[b] * D;
        const uint16_t *irows = idx_rows + (size_t)cu_new[b] * c->idx_dim;
        if (m == 0) { free(e); continue; }
        if (w_comp == NULL) {
            const int r = c->ratio;                    /* tokens per entry */
            if (p % r != 0) { raise_status(c, ORC_STATUS_ODD_ENTRY_APPEND); free(e); continue; }
            if (p / r + m > c->capacity) { raise_status(c, ORC_STATUS_OVERFLOW); free(e); continue; }
            for (int64_t q = 0; q < m; ++q)
                store_entry(c, b, p / r + q, rows + q * D, irows + q * c->idx_dim);
            c->n_tokens[b] = (int32_t)(p + (int64_t)r * m);
        } else {
            if ((p + m) / 2 > c->capacity) { raise_status(c, ORC_STATUS_OVERFLOW); free(e); continue; }
            for (int64_t q = 0; q < m; ++q) {
                int64_t pos = p + q;
                if (pos % 2 == 0) continue;            /* first half of a pair */
                const float *x_even = (q > 0) ? rows + (q - 1) * D : c->pending + (size_t)b * D;
                orc_compress_pair(w_comp, x_even, rows + q * D, D, e);
                store_entry(c, b, pos / 2, e, irows + q * c->idx_dim);
            }
            if ((p + m) % 2 != 0)
                memcpy(c->pending + (size_t)b * D, rows + (m - 1) * D, sizeof(float) * (size_t)D);
            c->n_tokens[b] = (int32_t)(p + m);
        }
        free(e);
    }
}

void orc_ced_project(const uint16_t *h, int64_t rows, int d_model, const uint16_t *w, int n_out,
                     float *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int n = 0; n < n_out; ++n) {
            double s = 0.0;
            for (int k = 0; k < d_model; ++k)
                s += orc_bf16_value(h[r * d_model + k]) * orc_bf16_value(w[(int64_t)n * d_model + k]);
            out[r * n_out + n] = (float)s;
        }
    }
}

void orc_swa_append(uint16_t *ring, int batch, int W, int dim, const float *rows,
                    const int32_t *cu_new, const int32_t *end_pos)
{
    for (int b = 0; b < batch; ++b) {
        int64_t m = cu_new[b + 1] - cu_new[b];
        for (int64_t q = 0; q < m; ++q) {
            int64_t pos = (int64_t)end_pos[b] - m + q;
            if (pos < 0 || pos < (int64_t)end_pos[b] - W) continue;
            const float *x = rows + (size_t)(cu_new[b] + q) * dim;
            uint16_t *dst = ring + ((size_t)b * W + (size_t)(pos % W)) * dim;
            for (int d = 0; d < dim; ++d) dst[d] = orc_bf16_from_f32(x[d]);
        }
    }
}

/* ------------------------------------------------------------ indexer */

void orc_indexer_scores(const uint16_t *keys, int64_t E, int idx_dim,
                        const uint16_t *q, int heads, const float *head_w,
                        double *scores)
{
    for (int64_t j = 0; j < E; ++j) {
        double s = 0.0;
        for (int h = 0; h < heads; ++h) {
            double dot = 0.0;
            for (int d = 0; d < idx_dim; ++d)
                dot += orc_bf16_value(q[(size_t)h * idx_dim + d]) *
                       orc_bf16_value(keys[(size_t)j * idx_dim + d]);
            double w = head_w ? (double)head_w[h] : 1.0;
            s += w * (dot > 0.0 ? dot : 0.0);
        }
        scores[j] = s;
    }
}

typedef struct { double score; int64_t index; } scored;

static int by_score_then_index(const void *a, const void *b)
{
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->index < y->index) ? -1 : (x->index > y->index);
}

static int by_int32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

void orc_topk(const double *scores, int64_t E, int k, int32_t *out)
{
    scored *all = (scored *)malloc(sizeof(scored) * (size_t)(E > 0 ? E : 1));
    for (int64_t j = 0; j < E; ++j) { all[j].score = scores[j]; all[j].index = j; }
    qsort(all, (size_t)E, sizeof(scored), by_score_then_index);
    int64_t n = E < k ? E : k;
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)all[i].index;
    qsort(out, (size_t)n, sizeof(int32_t), by_int32);
    for (int64_t i = n; i < k; ++i) out[i] = -1;
    free(all);
}

/* The indexer scores of sequence b's first E entries from its stored keys:
 * bf16 keys directly, FP4 keys dequantised to their exact values. */
static void cache_scores(const orc_cache *c, int b, int64_t E, const uint16_t *q, int heads,
                         const float *head_w, double *scores)
{
    const int Di = c->idx_dim;
    if (c->idx_format != 1) {
        orc_indexer_scores(c->idx_keys + (size_t)b * c->capacity * Di, E, Di, q, heads, head_w, scores);
        return;
    }
    double *k = (double *)malloc(sizeof(double) * (size_t)Di);
    for (int64_t j = 0; j < E; ++j) {
        size_t row = (size_t)b * c->capacity + (size_t)j;
        orc_dequantize_mx16((const uint8_t *)c->idx_keys + row * (Di / 2), c->idx_scales + row * (Di / 16), Di, k);
        double sc = 0.0;
        for (int h = 0; h < heads; ++h) {
            double dot = 0.0;
            for (int d = 0; d < Di; ++d) dot += orc_bf16_value(q[(size_t)h * Di + d]) * k[d];
            double w = head_w ? (double)head_w[h] : 1.0;
            sc += w * (dot > 0.0 ? dot : 0.0);
        }
        scores[j] = sc;
    }
    free(k);
}

static int64_t entries_of(const orc_cache *c, int b)
{
    int64_t e = c->n_tokens[b] / c->ratio;
    if (e < 0) e = 0;
    if (e > c->capacity) e = c->capacity;
    return e;
}

void orc_indexer_topk(const orc_cache *c, const uint16_t *q, int heads,
                      const float *head_w, int k, int32_t *out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < c->batch; ++b) {
        int64_t E = entries_of(c, b);
        double *s = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
        cache_scores(c, b, E, q + (size_t)b * heads * c->idx_dim, heads,
                     head_w ? head_w + (size_t)b * heads : NULL, s);
        orc_topk(s, E, k, out + (size_t)b * k);
        free(s);
    }
}

/* ------------------------------------------------------------ candidate pool */

void orc_pool_blocks(const double *scores, int64_t E, int block, int nb, int32_t *pool)
{
    int64_t nblocks = E > 0 ? (E + block - 1) / block : 0;
    double *bmax = (double *)malloc(sizeof(double) * (size_t)(nblocks > 0 ? nblocks : 1));
    for (int64_t i = 0; i < nblocks; ++i) {
        double m = -INFINITY;
        for (int64_t j = i * block; j < (i + 1) * block && j < E; ++j)
            if (scores[j] > m) m = scores[j];
        bmax[i] = m;
    }
    orc_topk(bmax, nblocks, nb, pool);
    free(bmax);
}

void orc_topk_in_pool(const double *scores, int64_t E, const int32_t *pool, int nb, int block,
                      int k, int32_t *out)
{
    /* the pooled entries in ascending order, and their scores */
    int64_t *ent = (int64_t *)malloc(sizeof(int64_t) * (size_t)nb * block + 1);
    double *sub = (double *)malloc(sizeof(double) * (size_t)nb * block + 1);
    int64_t n = 0;
    for (int i = 0; i < nb; ++i) {
        if (pool[i] < 0) continue;
        for (int64_t j = (int64_t)pool[i] * block; j < ((int64_t)pool[i] + 1) * block && j < E; ++j) {
            ent[n] = j;
            sub[n] = scores[j];
            ++n;
        }
    }
    /* positions in `sub` ascend with the entry index, so the top-k tie rule
     * on positions is the tie rule on entries */
    orc_topk(sub, n, k, out);
    for (int i = 0; i < k; ++i)
        if (out[i] >= 0) out[i] = (int32_t)ent[out[i]];
    free(ent);
    free(sub);
}

void orc_indexer_pool(const orc_cache *c, const uint16_t *q, int heads, const float *head_w,
                      int block, int nb, int32_t *pool)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < c->batch; ++b) {
        int64_t E = entries_of(c, b);
        double *s = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
        cache_scores(c, b, E, q + (size_t)b * heads * c->idx_dim, heads,
                     head_w ? head_w + (size_t)b * heads : NULL, s);
        orc_pool_blocks(s, E, block, nb, pool + (size_t)b * nb);
        free(s);
    }
}

void orc_indexer_topk_in_pool(const orc_cache *c, const uint16_t *q, int heads,
                              const float *head_w, const int32_t *pool, int nb, int block, int k,
                              int32_t *out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < c->batch; ++b) {
        int64_t E = entries_of(c, b);
        double *s = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
        cache_scores(c, b, E, q + (size_t)b * heads * c->idx_dim, heads,
                     head_w ? head_w + (size_t)b * heads : NULL, s);
        orc_topk_in_pool(s, E, pool + (size_t)b * nb, nb, block, k, out + (size_t)b * k);
        free(s);
    }
}

/* ------------------------------------------------------------ attention */

void orc_sparse_attn(const orc_cache *c, const float *q, int heads, const int32_t *idx,
                     int k, const uint16_t *swa, int W, const int32_t *swa_len,
                     double scale, double *out, double *lse)
{
    const int D = c->dim, Dv = c->dim - c->rope_dim;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < c->batch; ++b) {
        int64_t E = entries_of(c, b);
        int64_t nswa = swa_len ? swa_len[b] : (c->n_tokens[b] < W ? c->n_tokens[b] : W);
        if (nswa < 0) nswa = 0;
        if (nswa > W) nswa = W;
        int64_t nk = 0, cap = k + nswa;
        double *K = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        double *V = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * Dv);
        /* keys from the compressed cache: dequantise (exact in fp64) */
        for (int t = 0; t < k; ++t) {
            int64_t j = idx[(size_t)b * k + t];
            if (j < 0 || j >= E) continue;
            size_t row = (size_t)b * c->capacity + (size_t)j;
            if (c->k_format == 1) {
                orc_dequantize_mx16(c->k_codes + row * (D / 2), (const uint8_t *)c->k_scales + row * (D / 16),
                                    D, K + nk * D);
                if (c->v_group > 0)
                    orc_dequantize_mx16(c->v_codes + row * (Dv / 2),
                                        (const uint8_t *)c->v_scales + row * (Dv / 16), Dv, V + nk * Dv);
                else
                    memcpy(V + nk * Dv, K + nk * D, sizeof(double) * (size_t)Dv);
            } else {
                orc_dequantize_row(c->k_codes + row * (D / 2), c->k_scales + row * (D / c->k_group),
                                   D, c->k_group, K + nk * D);
                if (c->v_group > 0)
                    orc_dequantize_row(c->v_codes + row * (Dv / 2),
                                       c->v_scales + row * (Dv / c->v_group), Dv, c->v_group,
                                       V + nk * Dv);
                else
                    memcpy(V + nk * Dv, K + nk * D, sizeof(double) * (size_t)Dv);
            }
            ++nk;
        }
        /* keys from the sliding window (bf16 or FP8 rows; values are the first Dv dims) */
        for (int64_t s = 0; s < nswa; ++s) {
            if (c->swa_format == 1) {
                const uint8_t *r = (const uint8_t *)swa + ((size_t)b * W + (size_t)s) * D;
                for (int d = 0; d < D; ++d) K[nk * D + d] = orc_e4m3_value(r[d]);
            } else {
                const uint16_t *r = swa + ((size_t)b * W + (size_t)s) * D;
                for (int d = 0; d < D; ++d) K[nk * D + d] = orc_bf16_value(r[d]);
            }
            memcpy(V + nk * Dv, K + nk * D, sizeof(double) * (size_t)Dv);
            ++nk;
        }
        double *logit = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        for (int h = 0; h < heads; ++h) {
            const float *qh = q + ((size_t)b * heads + h) * D;
            double *o = out + ((size_t)b * heads + h) * Dv;
            for (int d = 0; d < Dv; ++d) o[d] = 0.0;
            if (nk == 0) { lse[(size_t)b * heads + h] = -INFINITY; continue; }
            double mx = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += (double)qh[d] * K[j * D + d];
                logit[j] = scale * dot;
                if (logit[j] > mx) mx = logit[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                double p = exp(logit[j] - mx);
                l += p;
                for (int d = 0; d < Dv; ++d) o[d] += p * V[j * Dv + d];
            }
            for (int d = 0; d < Dv; ++d) o[d] /= l;
            lse[(size_t)b * heads + h] = mx + log(l);
        }
        free(logit);
        free(K);
        free(V);
    }
}
