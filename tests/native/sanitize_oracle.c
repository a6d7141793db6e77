/*
 * Host sanitizer run of the CPU oracle.
 *
 * Built together with oracle/cskv_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (see tests/test_oracle_pins.py), this driver
 * calls every oracle entry point on small caches whose planes are allocated
 * at exactly the size the cache layout gives, so that a read or write one
 * element past any plane, an index computed in an overflowing signed type or
 * an out-of-range shift or float-to-int conversion stops the run.  The cases
 * cover the edges the oracle handles explicitly: empty sequences, a sequence
 * at capacity whose next token overflows, odd token counts (the pending
 * token), k larger than the entry count, indices that are -1 or past the
 * entry count, an empty window, pools with padded slots, every storage
 * format (fp32 scales at groups 16/32/64 with and without a value plane,
 * 16-channel E8M0 scales, bf16 and FP4 indexer keys, bf16 and FP8 window
 * rings) and every finite special value of the scalar encoders.
 *
 * It checks no values: the pins of the other tests do that.  It prints one
 * line per configuration and "ok" at the end; any sanitizer report ends the
 * process with a non-zero status.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/cskv_oracle.h"

static uint64_t rng_state = 0x243F6A8885A308D3ull;

static uint32_t next_u32(void)
{
    /* xorshift64* (Vigna), upper 32 bits */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static float uniform(float lo, float hi)
{
    return lo + (hi - lo) * (float)(next_u32() >> 8) * (1.0f / 16777216.0f);
}

static void *alloc(size_t n)
{
    /* exact size, never zero bytes, so any overrun lands in a redzone */
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(3); }
    memset(p, 0, n ? n : 1);
    return p;
}

typedef struct {
    int k_group, v_group, idx_format, k_format, swa_format, idx_dim;
} config;

static orc_cache make_cache(const config *f, int batch, int cap)
{
    orc_cache c;
    memset(&c, 0, sizeof c);
    const int D = 576, R = 64, Dv = D - R;
    c.batch = batch;
    c.capacity = cap;
    c.dim = D;
    c.rope_dim = R;
    c.k_group = f->k_group;
    c.v_group = f->v_group;
    c.idx_dim = f->idx_dim;
    c.idx_format = f->idx_format;
    c.swa_format = f->swa_format;
    c.k_format = f->k_format;
    c.ratio = 2;
    const size_t rows = (size_t)batch * cap;
    c.k_codes = alloc(rows * (D / 2));
    c.k_scales = alloc(f->k_format == 1 ? rows * (D / 16) : rows * (D / f->k_group) * sizeof(float));
    if (f->v_group > 0) {
        c.v_codes = alloc(rows * (Dv / 2));
        c.v_scales = alloc(f->k_format == 1 ? rows * (Dv / 16) : rows * (Dv / f->v_group) * sizeof(float));
    }
    if (f->idx_format == 1) {
        c.idx_keys = alloc(rows * (f->idx_dim / 2));
        c.idx_scales = alloc(rows * (f->idx_dim / 16));
    } else {
        c.idx_keys = alloc(rows * f->idx_dim * sizeof(uint16_t));
    }
    c.n_tokens = alloc(sizeof(int32_t) * batch);
    c.pending = alloc(sizeof(float) * (size_t)batch * D);
    c.status = alloc(sizeof(int32_t));
    return c;
}

static void free_cache(orc_cache *c)
{
    free(c->k_codes); free(c->k_scales); free(c->v_codes); free(c->v_scales);
    free(c->idx_keys); free(c->idx_scales); free(c->n_tokens); free(c->pending); free(c->status);
}

static float *random_rows(size_t n, float amp)
{
    float *x = alloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) {
        float v = uniform(-amp, amp);
        /* a few exact zeros and tiny values, so zero groups and subnormal
         * quotients occur */
        uint32_t r = next_u32() % 64;
        if (r == 0) v = 0.0f;
        else if (r == 1) v = -0.0f;
        else if (r == 2) v *= 1e-30f;
        x[i] = v;
    }
    return x;
}

static uint16_t *random_bf16(size_t n)
{
    uint16_t *x = alloc(sizeof(uint16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) x[i] = orc_bf16_from_f32((float)((int)(next_u32() % 9) - 4));
    return x;
}

static int32_t *prefix(const int *m, int batch)
{
    int32_t *cu = alloc(sizeof(int32_t) * (batch + 1));
    for (int b = 0; b < batch; ++b) cu[b + 1] = cu[b] + m[b];
    return cu;
}

/* tokens of one call: rows fp32 [total][576], indexer rows bf16 [total][idx_dim] */
static void append_tokens(orc_cache *c, const float *w, const int *m, void *ring, int W)
{
    const int B = c->batch, D = c->dim;
    int32_t *cu = prefix(m, B);
    const size_t total = (size_t)cu[B];
    float *rows = random_rows(total * D, 3.0f);
    uint16_t *irows = random_bf16(total * c->idx_dim);
    orc_kv_append(c, rows, cu, w, irows);
    int32_t *end = alloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b) end[b] = c->n_tokens[b];
    if (c->swa_format == 1) orc_swa_append_fp8(ring, B, W, D, rows, cu, end);
    else orc_swa_append(ring, B, W, D, rows, cu, end);
    free(end); free(rows); free(irows); free(cu);
}

static void append_entries(orc_cache *c, const int *m)
{
    const int B = c->batch, D = c->dim;
    int32_t *cu = prefix(m, B);
    const size_t total = (size_t)cu[B];
    float *rows = random_rows(total * D, 8.0f);
    uint16_t *irows = random_bf16(total * c->idx_dim);
    orc_kv_append(c, rows, cu, NULL, irows);
    free(rows); free(irows); free(cu);
}

static void read_paths(orc_cache *c, const void *ring, int W)
{
    const int B = c->batch, H = 3, Hq = 4, D = c->dim, Dv = D - c->rope_dim;
    uint16_t *q = random_bf16((size_t)B * H * c->idx_dim);
    float *hw = alloc(sizeof(float) * B * H);
    for (int i = 0; i < B * H; ++i) hw[i] = uniform(0.0f, 2.0f);
    for (int k = 1; k <= 64; k *= 4) {
        int32_t *idx = alloc(sizeof(int32_t) * B * k);
        orc_indexer_topk(c, q, H, NULL, k, idx);
        orc_indexer_topk(c, q, H, hw, k, idx);
        const int block = 4, nb = 3;
        int32_t *pool = alloc(sizeof(int32_t) * B * nb);
        orc_indexer_pool(c, q, H, hw, block, nb, pool);
        orc_indexer_topk_in_pool(c, q, H, hw, pool, nb, block, k, idx);
        /* attention over the selection with a -1 and an index past the count
         * planted, the window at its natural length and at given lengths */
        if (k > 1) { idx[0] = -1; idx[k - 1] = c->capacity + 5; }
        float *qa = random_rows((size_t)B * Hq * D, 1.0f);
        double *out = alloc(sizeof(double) * B * Hq * Dv), *lse = alloc(sizeof(double) * B * Hq);
        orc_sparse_attn(c, qa, Hq, idx, k, ring, W, NULL, 0.04, out, lse);
        int32_t *len = alloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b) len[b] = (b * 7) % (W + 3) - 1;   /* -1, in range, past W */
        orc_sparse_attn(c, qa, Hq, idx, k, ring, W, len, 0.04, out, lse);
        free(len); free(out); free(lse); free(qa); free(pool); free(idx);
    }
    free(q); free(hw);
}

static void run_config(const config *f)
{
    const int B = 4, cap = 40, W = 8, D = 576;
    printf("config: k_group %d v_group %d idx_format %d k_format %d swa_format %d idx_dim %d\n",
           f->k_group, f->v_group, f->idx_format, f->k_format, f->swa_format, f->idx_dim);
    fflush(stdout);
    float *w = random_rows((size_t)D * 2 * D, 0.03f);
    orc_cache c = make_cache(f, B, cap);
    void *ring = alloc((size_t)B * W * D * (f->swa_format == 1 ? 1 : 2));
    /* prefill: an empty sequence, an odd count, capacity exactly, one short of it */
    const int pre[4] = {0, 13, 2 * cap, 2 * cap - 1};
    append_tokens(&c, w, pre, ring, W);
    read_paths(&c, ring, W);
    /* three decode steps: pending tokens, completions, the overflow of sequence 2 */
    const int one[4] = {1, 1, 1, 1};
    for (int s = 0; s < 3; ++s) {
        append_tokens(&c, w, one, ring, W);
        read_paths(&c, ring, W);
    }
    /* entries mode on a second cache, including an odd-token sequence */
    orc_cache e = make_cache(f, B, cap);
    const int ent[4] = {0, 5, cap, cap + 1};
    append_entries(&e, ent);
    e.n_tokens[1] += 1;
    const int more[4] = {1, 1, 0, 1};
    append_entries(&e, more);
    read_paths(&e, ring, W);
    free_cache(&e);
    free_cache(&c);
    free(ring);
    free(w);
}

static void scalars(void)
{
    const float special[] = {0.0f, -0.0f, FLT_MIN, -FLT_MIN, 1e-45f, -1e-45f, FLT_MAX, -FLT_MAX,
                             0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 6.0f, 7.0f, 448.0f,
                             464.0f, 1e30f, -1e30f, 3.3895314e38f, 0.001953125f, 0.0009765625f};
    unsigned acc = 0;
    for (size_t i = 0; i < sizeof special / sizeof special[0]; ++i) {
        acc += orc_e2m1_encode(special[i]);
        acc += orc_bf16_from_f32(special[i]);
        acc += orc_e4m3_encode(special[i]);
    }
    for (unsigned v = 0; v < 16; ++v) acc += (unsigned)orc_e2m1_value(v);
    for (unsigned v = 0; v < 256; ++v) {
        acc += isfinite(orc_e8m0_value((uint8_t)v));
        acc += isfinite(orc_e4m3_value((uint8_t)v));
    }
    for (unsigned v = 0; v < 65536; ++v) acc += isfinite(orc_bf16_value((uint16_t)v));
    /* rows of special values through every quantiser and its inverse */
    const int n = 64;
    float *x = alloc(sizeof(float) * n);
    uint16_t *xb = alloc(sizeof(uint16_t) * n);
    for (int i = 0; i < n; ++i) {
        x[i] = special[i % (int)(sizeof special / sizeof special[0])] * ((i & 1) ? -1.0f : 1.0f);
        xb[i] = orc_bf16_from_f32(i < 16 ? 0.0f : x[i] * 1e-30f);
    }
    uint8_t *codes = alloc(n / 2), *s8 = alloc(n / 16);
    double *back = alloc(sizeof(double) * n);
    for (int g = 16; g <= 64; g *= 2) {
        float *sc = alloc(sizeof(float) * (n / g));
        orc_quantize_row(x, n, g, codes, sc);
        orc_dequantize_row(codes, sc, n, g, back);
        free(sc);
    }
    orc_quantize_mx16_f32(x, n, codes, s8);
    orc_dequantize_mx16(codes, s8, n, back);
    orc_quantize_mx16(xb, n, codes, s8);
    orc_dequantize_mx16(codes, s8, n, back);
    /* top-k on empty input, fewer scores than k, all scores tied */
    double *sc = alloc(sizeof(double) * 16);
    int32_t *out = alloc(sizeof(int32_t) * 32);
    orc_topk(sc, 0, 4, out);
    orc_topk(sc, 16, 32, out);
    int32_t *pool = alloc(sizeof(int32_t) * 8);
    orc_pool_blocks(sc, 16, 3, 8, pool);
    orc_topk_in_pool(sc, 16, pool, 8, 3, 32, out);
    orc_pool_blocks(sc, 0, 3, 8, pool);
    orc_topk_in_pool(sc, 0, pool, 8, 3, 4, out);
    /* CED projection with ragged sizes, and the byte accounting */
    uint16_t *h = random_bf16(3 * 40), *wp = random_bf16(5 * 40);
    float *proj = alloc(sizeof(float) * 3 * 5);
    orc_ced_project(h, 3, 40, wp, 5, proj);
    orc_ced_project(h, 0, 40, wp, 5, proj);
    const int ratio[4] = {2, 2, 2, 1};
    acc += (unsigned)orc_kv_bytes(95, 1, 128, 128, 2);
    acc += (unsigned)orc_fp4_row_bytes(512, 16, 1.0);
    acc += (unsigned)orc_global_kv_per_token(4, ratio, 288.0, 72.0);
    printf("scalars: %u\n", acc);
    free(h); free(wp); free(proj); free(pool); free(out); free(sc);
    free(back); free(codes); free(s8); free(x); free(xb);
}

int main(void)
{
    scalars();
    const config configs[] = {
        {64, 0, 0, 0, 0, 128},
        {32, 128, 1, 0, 1, 128},
        {16, 16, 1, 1, 0, 64},
        {16, 0, 0, 1, 1, 64},
        {64, 64, 1, 0, 0, 64},
    };
    for (size_t i = 0; i < sizeof configs / sizeof configs[0]; ++i) run_config(&configs[i]);
    printf("ok\n");
    return 0;
}
