// api.cpp -- the C ABI: argument checks, launch order, timers.
//
// Sources cited as [P2] (page title, then the section):
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "cskv.h"
#include "launch.hpp"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(CSKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, code, ...)              \
    do {                                      \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

int check_cache(const cskv_cache *c)
{
    REQUIRE(c, CSKV_EINVAL, "cache descriptor is NULL");
    REQUIRE(c->batch >= 1 && c->batch <= 65535, CSKV_EINVAL, "batch %d out of [1, 65535]", c->batch);
    REQUIRE(c->capacity >= 1 && c->capacity <= (1 << 26), CSKV_EINVAL,
            "capacity %d out of [1, 2^26]", c->capacity);
    REQUIRE(c->dim == 576 && c->rope_dim == 64, CSKV_EUNSUPPORTED,
            "dim %d / rope_dim %d: only 576 / 64 are built", c->dim, c->rope_dim);
    REQUIRE(c->k_format == CSKV_KV_F32 || c->k_format == CSKV_KV_MX16, CSKV_EUNSUPPORTED,
            "k_format %d: CSKV_KV_F32 or CSKV_KV_MX16", c->k_format);
    if (c->k_format == CSKV_KV_MX16) {
        REQUIRE(c->k_group == 16 && (c->v_group == 0 || c->v_group == 16), CSKV_EUNSUPPORTED,
                "k_group %d / v_group %d: CSKV_KV_MX16 takes 16 / 0 or 16", c->k_group, c->v_group);
    } else {
        REQUIRE(c->k_group == 32 || c->k_group == 64, CSKV_EUNSUPPORTED,
                "k_group %d: 32 or 64 supported (must divide 576)", c->k_group);
        REQUIRE(c->v_group == 0 || c->v_group == 32 || c->v_group == 64 || c->v_group == 128,
                CSKV_EUNSUPPORTED, "v_group %d: 0, 32, 64 or 128 supported", c->v_group);
    }
    REQUIRE(c->idx_dim == 64 || c->idx_dim == 128, CSKV_EUNSUPPORTED,
            "idx_dim %d: 64 or 128 supported", c->idx_dim);
    REQUIRE(c->k_codes && c->k_scales && c->idx_keys && c->n_tokens && c->pending && c->status,
            CSKV_EINVAL, "cache plane pointer is NULL");
    REQUIRE((c->v_group > 0) == (c->v_codes != nullptr) && (c->v_group > 0) == (c->v_scales != nullptr),
            CSKV_EINVAL, "value plane pointers must be set exactly when v_group > 0");
    REQUIRE(c->idx_format == CSKV_IDX_BF16 || c->idx_format == CSKV_IDX_FP4, CSKV_EUNSUPPORTED,
            "idx_format %d: CSKV_IDX_BF16 or CSKV_IDX_FP4", c->idx_format);
    REQUIRE((c->idx_format == CSKV_IDX_FP4) == (c->idx_scales != nullptr), CSKV_EINVAL,
            "idx_scales must be set exactly for CSKV_IDX_FP4");
    REQUIRE(!c->idx_scales || aligned(c->idx_scales, 16), CSKV_EINVAL, "idx_scales must be 16-byte aligned");
    REQUIRE(c->swa_format == CSKV_SWA_BF16 || c->swa_format == CSKV_SWA_FP8, CSKV_EUNSUPPORTED,
            "swa_format %d: CSKV_SWA_BF16 or CSKV_SWA_FP8", c->swa_format);
    REQUIRE(c->ratio == 1 || c->ratio == 2, CSKV_EUNSUPPORTED, "ratio %d: 1 or 2 tokens per entry", c->ratio);
    REQUIRE(c->page_size >= 0, CSKV_EINVAL, "page_size %d < 0", c->page_size);
    if (c->page_size > 0) {
        REQUIRE(c->page_size >= 64 && (c->page_size & (c->page_size - 1)) == 0, CSKV_EUNSUPPORTED,
                "page_size %d: a power of two of at least 64", c->page_size);
        REQUIRE(c->max_pages >= 1 && (int64_t)c->max_pages * c->page_size == c->capacity, CSKV_EINVAL,
                "capacity %d must equal max_pages %d x page_size %d", c->capacity, c->max_pages, c->page_size);
        REQUIRE(c->n_pages >= 1 && c->block_table && aligned(c->block_table, 4), CSKV_EINVAL,
                "a paged cache needs n_pages >= 1 and a 4-byte aligned block table");
        REQUIRE((int64_t)c->n_pages * c->page_size * (c->dim / 2) < ((int64_t)1 << 31), CSKV_EUNSUPPORTED,
                "paged planes of %d pages x %d entries pass 2 GiB", c->n_pages, c->page_size);
    }
    REQUIRE(aligned(c->k_codes, 16) && aligned(c->k_scales, 16) && aligned(c->idx_keys, 16) &&
                aligned(c->n_tokens, 16) && aligned(c->pending, 16) && aligned(c->status, 4) &&
                (!c->v_codes || aligned(c->v_codes, 16)) && (!c->v_scales || aligned(c->v_scales, 16)),
            CSKV_EINVAL, "cache planes must be 16-byte aligned");
    return CSKV_OK;
}

int check_rows(const void *rows, const int32_t *cu_new, int32_t total_new, int32_t batch)
{
    REQUIRE(total_new >= 0, CSKV_EINVAL, "total_new %d < 0", total_new);
    REQUIRE(total_new == 0 || rows, CSKV_EINVAL, "rows are NULL");
    REQUIRE(rows == nullptr || aligned(rows, 16), CSKV_EINVAL, "rows must be 16-byte aligned");
    REQUIRE(cu_new || total_new == batch, CSKV_EINVAL,
            "cu_new NULL needs total_new == batch (%d != %d)", total_new, batch);
    return CSKV_OK;
}

int topk_args(const cskv_cache *c, const uint16_t *q_idx, int32_t heads, int32_t k,
              const int32_t *out_idx, const void *ws, size_t ws_bytes)
{
    REQUIRE(q_idx && aligned(q_idx, 16), CSKV_EINVAL, "q_idx NULL or not 16-byte aligned");
    REQUIRE(heads >= 1 && heads <= 64, CSKV_EUNSUPPORTED, "n_idx_heads %d out of [1, 64]", heads);
    REQUIRE(k >= 1 && k <= 2048, CSKV_EUNSUPPORTED, "k %d out of [1, 2048]", k);
    REQUIRE(out_idx, CSKV_EINVAL, "out_idx is NULL");
    const size_t need = cskv::topk_workspace(*c, k).total;
    REQUIRE(ws && aligned(ws, 256), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return CSKV_OK;
}

int attn_shape(int32_t heads, int32_t k, int32_t window)
{
    REQUIRE(heads >= 16 && heads <= 1024 && heads % 16 == 0, CSKV_EUNSUPPORTED,
            "n_heads %d: a multiple of 16 in [16, 1024]", heads);
    REQUIRE(k >= 1 && k <= 2048, CSKV_EUNSUPPORTED, "k %d out of [1, 2048]", k);
    REQUIRE(window >= 1 && window <= 1024, CSKV_EUNSUPPORTED, "window %d out of [1, 1024]", window);
    return CSKV_OK;
}

int attn_args(const cskv_cache *c, const float *q, int32_t heads, const int32_t *idx, bool need_idx,
              int32_t k, const uint16_t *swa, int32_t window, const float *out, const float *lse,
              const void *ws, size_t ws_bytes)
{
    REQUIRE(q && out && (idx || !need_idx), CSKV_EINVAL, "q, idx or out is NULL");
    int rc = attn_shape(heads, k, window);
    if (rc) return rc;
    REQUIRE(c->capacity <= (1 << 23), CSKV_EUNSUPPORTED,
            "capacity %d: attention supports at most 2^23 entries per sequence", c->capacity);
    REQUIRE(aligned(q, 16) && aligned(out, 16) && (!idx || aligned(idx, 4)) && (!lse || aligned(lse, 4)),
            CSKV_EINVAL, "q and out must be 16-byte aligned");
    REQUIRE(swa && aligned(swa, 16), CSKV_EINVAL, "window ring NULL or not 16-byte aligned");
    const size_t need = cskv::attn_plan(*c, heads, k, window).ws_bytes;
    REQUIRE(need == 0 || (ws && aligned(ws, 256)), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return CSKV_OK;
}

int pool_args(const cskv_cache *c, int32_t k, int32_t pool_blocks, int32_t pool_block)
{
    REQUIRE(pool_block == 2 || pool_block == 4 || pool_block == 8 || pool_block == 16, CSKV_EUNSUPPORTED,
            "pool_block %d: 2, 4, 8 or 16", pool_block);
    REQUIRE(pool_blocks >= 1 && pool_blocks <= 2048, CSKV_EUNSUPPORTED, "pool_blocks %d out of [1, 2048]",
            pool_blocks);
    REQUIRE((int64_t)pool_blocks * pool_block >= (int64_t)k + pool_block, CSKV_EUNSUPPORTED,
            "pool of %d x %d positions too small for k = %d", pool_blocks, pool_block, k);
    (void)c;
    return CSKV_OK;
}

// Layer-group workspace: the candidate pool (when used) at offset 0, then a
// region shared in turn by the append, each layer's top-k and attention.  A
// decode step whose append rides on the first top-k keeps the compressed
// entry and its cache rows past the top-k's (and the pool build's) part of
// that region, from the append's head kernel until the top-k's last launch.
size_t group_pool_bytes(const cskv_cache &c, int pool_blocks)
{
    return pool_blocks > 0 ? ((size_t)c.batch * pool_blocks * sizeof(int32_t) + 255) / 256 * 256 : 0;
}

static size_t group_carry_off(const cskv_cache &c, int k, int pool_blocks, int pool_block)
{
    size_t off = cskv::topk_workspace(c, k).total;
    if (pool_blocks > 0) off = std::max(off, cskv::pool_workspace(c, k, pool_blocks, pool_block).build_total);
    return (off + 255) / 256 * 256;
}

size_t group_ws_bytes(const cskv_cache &c, int heads, int k, int window, int pool_blocks, int pool_block)
{
    size_t need = cskv::topk_workspace(c, k).total;
    if (pool_blocks > 0) {
        const cskv::PoolWorkspace pw = cskv::pool_workspace(c, k, pool_blocks, pool_block);
        need = std::max(need, std::max(pw.build_total, pw.inpool_total));
    }
    need = std::max(need, cskv::attn_plan(c, heads, k, window).ws_bytes);
    need = std::max(need, cskv::append_workspace_bytes(c.batch));   // one new token per sequence
    if (cskv::topk_carries_entry(c, k))
        need = std::max(need, group_carry_off(c, k, pool_blocks, pool_block) + cskv::deferred_entry_bytes(c.batch));
    need = std::max(need, (size_t)256);
    return group_pool_bytes(c, pool_blocks) + need;
}

// ---------------------------------------------------------------- scratch

// The workspace of cskv_layer_group_decode_noalloc: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// uses its name as an address: each device's address is looked up once with
// hipGetSymbolAddress (with that device current) and kept here.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[CSKV_NOALLOC_SCRATCH_BYTES];
void *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_of_current_device(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    REQUIRE(dev >= 0 && dev < kMaxDevices, CSKV_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        REQUIRE(p && aligned(p, 256), CSKV_EHIP, "scratch address not 256-byte aligned");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CSKV_OK;
}

// ---------------------------------------------------------------- timers

struct Timer {
    bool on = false, paused = false;
    int max = 0, count = 0;
    std::vector<hipEvent_t> start, stop;
};
Timer g_timers[8];

void free_timer(Timer &T)
{
    for (auto e : T.start) (void)hipEventDestroy(e);
    for (auto e : T.stop) (void)hipEventDestroy(e);
    T = Timer();
}

}  // namespace

namespace cskv {
TimedLaunch timer_take(int kind)
{
    Timer &T = g_timers[kind];
    TimedLaunch t;
    if (T.on && !T.paused && T.count < T.max) {
        t.start = T.start[T.count];
        t.stop = T.stop[T.count];
        ++T.count;
    }
    return t;
}
}  // namespace cskv

extern "C" {

const char *cskv_last_error(void) { return g_error.c_str(); }

size_t cskv_entry_bytes(int32_t dim, int32_t rope_dim, int32_t k_group, int32_t v_group,
                        int32_t idx_dim)
{
    if (dim <= 0 || k_group <= 0 || dim % k_group) return 0;
    size_t b = (size_t)dim / 2 + 4 * (size_t)(dim / k_group) + 2 * (size_t)idx_dim;
    if (v_group > 0) {
        const int dv = dim - rope_dim;
        if (dv <= 0 || dv % v_group) return 0;
        b += (size_t)dv / 2 + 4 * (size_t)(dv / v_group);
    }
    return b;
}

size_t cskv_cache_entry_bytes(const cskv_cache *cache)
{
    if (check_cache(cache) != CSKV_OK) return 0;
    const cskv_cache &c = *cache;
    const size_t per_scale = c.k_format == CSKV_KV_MX16 ? 1 : 4;
    size_t b = (size_t)c.dim / 2 + per_scale * (size_t)(c.dim / c.k_group);
    if (c.v_group > 0) {
        const int dv = c.dim - c.rope_dim;
        b += (size_t)dv / 2 + per_scale * (size_t)(dv / c.v_group);
    }
    b += c.idx_format == CSKV_IDX_FP4 ? (size_t)c.idx_dim / 2 + (size_t)c.idx_dim / 16 : 2 * (size_t)c.idx_dim;
    return b;
}

size_t cskv_workspace_bytes(const cskv_cache *cache, int32_t op, int32_t n_heads, int32_t k,
                            int32_t window)
{
    if (check_cache(cache) != CSKV_OK) return 0;
    size_t topk = 0, attn = 0;
    if (op == CSKV_OP_INDEXER_TOPK || op == CSKV_OP_LAYER_GROUP) {
        if (k < 1 || k > 2048) {
            fail(CSKV_EUNSUPPORTED, "k %d out of [1, 2048]", k);
            return 0;
        }
        topk = cskv::topk_workspace(*cache, k).total;
    }
    if (op == CSKV_OP_SPARSE_ATTN || op == CSKV_OP_LAYER_GROUP) {
        if (attn_shape(n_heads, k, window) != CSKV_OK) return 0;
        attn = cskv::attn_plan(*cache, n_heads, k, window).ws_bytes;
    }
    if (op < CSKV_OP_INDEXER_TOPK || op > CSKV_OP_LAYER_GROUP) {
        fail(CSKV_EINVAL, "unknown workspace op %d", op);
        return 0;
    }
    if (op == CSKV_OP_LAYER_GROUP) return group_ws_bytes(*cache, n_heads, k, window, 0, 0);
    const size_t need = topk > attn ? topk : attn;
    return need > 256 ? need : 256;
}

size_t cskv_workspace_bytes_pool(const cskv_cache *cache, int32_t op, int32_t n_heads, int32_t k,
                                 int32_t window, int32_t pool_blocks, int32_t pool_block)
{
    if (op == CSKV_OP_INDEXER_POOL || op == CSKV_OP_INDEXER_IN_POOL) {
        if (check_cache(cache) != CSKV_OK) return 0;
        if (k < 1 || k > 2048) {
            fail(CSKV_EUNSUPPORTED, "k %d out of [1, 2048]", k);
            return 0;
        }
        if (pool_args(cache, k, pool_blocks, pool_block) != CSKV_OK) return 0;
        const cskv::PoolWorkspace pw = cskv::pool_workspace(*cache, k, pool_blocks, pool_block);
        return std::max(op == CSKV_OP_INDEXER_POOL ? pw.build_total : pw.inpool_total, (size_t)256);
    }
    if (op == CSKV_OP_LAYER_GROUP && pool_blocks != 0) {
        if (cskv_workspace_bytes(cache, op, n_heads, k, window) == 0) return 0;
        if (pool_args(cache, k, pool_blocks, pool_block) != CSKV_OK) return 0;
        return group_ws_bytes(*cache, n_heads, k, window, pool_blocks, pool_block);
    }
    return cskv_workspace_bytes(cache, op, n_heads, k, window);
}

size_t cskv_append_workspace_bytes(int32_t total_new, const float *w_comp)
{
    if (!w_comp || total_new <= 0) return 256;
    const size_t need = cskv::append_workspace_bytes(total_new);
    return need > 256 ? need : 256;
}

static int kv_append(const cskv_cache *cache, const float *tokens, const int32_t *cu_new,
                     int32_t total_new, const float *w_comp, const uint16_t *idx_rows,
                     void *ws, size_t ws_bytes, hipStream_t stream, bool mfma)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_rows(tokens, cu_new, total_new, cache->batch))) return rc;
    REQUIRE(total_new == 0 || (idx_rows && aligned(idx_rows, 4)), CSKV_EINVAL,
            "idx_rows NULL or not 4-byte aligned");
    REQUIRE(!w_comp || aligned(w_comp, 16), CSKV_EINVAL, "w_comp must be 16-byte aligned");
    REQUIRE(!w_comp || cache->ratio == 2, CSKV_EUNSUPPORTED, "the 2->1 compressor needs a ratio-2 cache");
    if (w_comp && total_new > 0) {
        const size_t need = cskv::append_workspace_bytes(total_new);
        REQUIRE(ws && aligned(ws, 256), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
        REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    }
    hipError_t e = cskv::launch_kv_append(*cache, tokens, cu_new, total_new, w_comp, idx_rows, ws, stream,
                                          nullptr, nullptr, 0, mfma);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "kv_append_fp4 launch");
}

int cskv_kv_append_fp4(const cskv_cache *cache, const float *tokens, const int32_t *cu_new,
                       int32_t total_new, const float *w_comp, const uint16_t *idx_rows,
                       void *ws, size_t ws_bytes, hipStream_t stream)
{
    return kv_append(cache, tokens, cu_new, total_new, w_comp, idx_rows, ws, ws_bytes, stream, false);
}

int cskv_kv_append_fp4_mfma(const cskv_cache *cache, const float *tokens, const int32_t *cu_new,
                            int32_t total_new, const float *w_comp, const uint16_t *idx_rows,
                            void *ws, size_t ws_bytes, hipStream_t stream)
{
    return kv_append(cache, tokens, cu_new, total_new, w_comp, idx_rows, ws, ws_bytes, stream, true);
}

int cskv_swa_append(uint16_t *ring, int32_t batch, int32_t window, int32_t dim, const float *rows,
                    const int32_t *cu_new, int32_t total_new, const int32_t *end_pos,
                    hipStream_t stream)
{
    REQUIRE(ring && aligned(ring, 16), CSKV_EINVAL, "ring NULL or not 16-byte aligned");
    REQUIRE(batch >= 1, CSKV_EINVAL, "batch %d < 1", batch);
    REQUIRE(window >= 1 && window <= (1 << 20), CSKV_EINVAL, "window %d out of [1, 2^20]", window);
    REQUIRE(dim > 0 && dim % 4 == 0, CSKV_EUNSUPPORTED, "dim %d must be a positive multiple of 4", dim);
    REQUIRE(end_pos, CSKV_EINVAL, "end_pos is NULL");
    int rc = check_rows(rows, cu_new, total_new, batch);
    if (rc) return rc;
    hipError_t e = cskv::launch_swa_append(ring, batch, window, dim, rows, cu_new, total_new, end_pos, stream);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "swa_append launch");
}

int cskv_swa_append_fp8(uint8_t *ring, int32_t batch, int32_t window, int32_t dim, const float *rows,
                        const int32_t *cu_new, int32_t total_new, const int32_t *end_pos,
                        hipStream_t stream)
{
    REQUIRE(ring && aligned(ring, 16), CSKV_EINVAL, "ring NULL or not 16-byte aligned");
    REQUIRE(batch >= 1, CSKV_EINVAL, "batch %d < 1", batch);
    REQUIRE(window >= 1 && window <= (1 << 20), CSKV_EINVAL, "window %d out of [1, 2^20]", window);
    REQUIRE(dim > 0 && dim % 16 == 0, CSKV_EUNSUPPORTED, "dim %d must be a positive multiple of 16", dim);
    REQUIRE(end_pos, CSKV_EINVAL, "end_pos is NULL");
    int rc = check_rows(rows, cu_new, total_new, batch);
    if (rc) return rc;
    hipError_t e = cskv::launch_swa_append(reinterpret_cast<uint16_t *>(ring), batch, window, dim, rows, cu_new,
                                           total_new, end_pos, stream, true);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "swa_append_fp8 launch");
}

int cskv_indexer_topk(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                      const float *head_w, int32_t k, int32_t *out_idx, float *out_scores, void *ws,
                      size_t ws_bytes, hipStream_t stream)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = topk_args(cache, q_idx, n_idx_heads, k, out_idx, ws, ws_bytes))) return rc;
    REQUIRE(!out_scores || aligned(out_scores, 4), CSKV_EINVAL, "out_scores must be 4-byte aligned");
    hipError_t e = cskv::launch_indexer_topk(*cache, q_idx, n_idx_heads, head_w, k, out_idx, ws, stream,
                                             nullptr, out_scores);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "indexer_topk launch");
}

int cskv_indexer_topk_pool(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                           const float *head_w, int32_t k, int32_t *out_idx, int32_t pool_blocks,
                           int32_t pool_block, int32_t *out_pool, void *ws, size_t ws_bytes,
                           hipStream_t stream)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = topk_args(cache, q_idx, n_idx_heads, k, out_idx, ws, ws_bytes))) return rc;
    if ((rc = pool_args(cache, k, pool_blocks, pool_block))) return rc;
    REQUIRE(out_pool, CSKV_EINVAL, "out_pool is NULL");
    const size_t need = cskv::pool_workspace(*cache, k, pool_blocks, pool_block).build_total;
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    const cskv::PoolBuild pb{pool_blocks, pool_block, out_pool};
    hipError_t e = cskv::launch_indexer_topk(*cache, q_idx, n_idx_heads, head_w, k, out_idx, ws, stream, &pb);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "indexer_topk_pool launch");
}

int cskv_indexer_topk_in_pool(const cskv_cache *cache, const uint16_t *q_idx, int32_t n_idx_heads,
                              const float *head_w, int32_t k, const int32_t *pool, int32_t pool_blocks,
                              int32_t pool_block, int32_t *out_idx, void *ws, size_t ws_bytes,
                              hipStream_t stream)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = pool_args(cache, k, pool_blocks, pool_block))) return rc;
    REQUIRE(q_idx && aligned(q_idx, 16), CSKV_EINVAL, "q_idx NULL or not 16-byte aligned");
    REQUIRE(n_idx_heads >= 1 && n_idx_heads <= 64, CSKV_EUNSUPPORTED, "n_idx_heads %d out of [1, 64]",
            n_idx_heads);
    REQUIRE(out_idx && pool && aligned(pool, 4), CSKV_EINVAL, "out_idx or pool is NULL");
    const size_t need = cskv::pool_workspace(*cache, k, pool_blocks, pool_block).inpool_total;
    REQUIRE(ws && aligned(ws, 256), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    hipError_t e = cskv::launch_indexer_topk_in_pool(*cache, q_idx, n_idx_heads, head_w, k, pool, pool_blocks,
                                                     pool_block, out_idx, ws, stream);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "indexer_topk_in_pool launch");
}

int cskv_sparse_attn_decode(const cskv_cache *cache, const float *q, int32_t n_heads,
                            const int32_t *idx, int32_t k, const uint16_t *swa, int32_t window,
                            const int32_t *swa_len, float softmax_scale, float *out, float *lse,
                            void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = attn_args(cache, q, n_heads, idx, true, k, swa, window, out, lse, ws, ws_bytes))) return rc;
    hipError_t e = cskv::launch_sparse_attn(*cache, q, n_heads, idx, k, swa, window, swa_len,
                                            softmax_scale, out, lse, ws, stream);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "sparse_attn_decode launch");
}

// Every check of one layer-group step, before anything is enqueued.
static int check_group(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                       const float *new_tokens, const float *w_comp, const uint16_t *new_idx_rows,
                       int32_t n_idx_heads, int32_t n_heads, int32_t k, int32_t window,
                       int32_t pool_blocks, int32_t pool_block, void *ws, size_t ws_bytes)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    REQUIRE(layers && n_layers >= 1 && n_layers <= 256, CSKV_EINVAL, "need 1..256 layers");
    REQUIRE(!new_tokens || (aligned(new_tokens, 16) && new_idx_rows), CSKV_EINVAL,
            "new_tokens must be 16-byte aligned and come with new_idx_rows");
    REQUIRE(!new_tokens || !w_comp || (aligned(w_comp, 16) && cache->ratio == 2), CSKV_EINVAL,
            "w_comp must be 16-byte aligned and the cache ratio 2");
    if (pool_blocks != 0 && (rc = pool_args(cache, k, pool_blocks, pool_block))) return rc;
    REQUIRE(ws && aligned(ws, 256), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    const size_t need = group_ws_bytes(*cache, n_heads, k, window, pool_blocks, pool_block);
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    const size_t pool_bytes = group_pool_bytes(*cache, pool_blocks);
    void *work = static_cast<char *>(ws) + pool_bytes;
    const size_t work_bytes = ws_bytes - pool_bytes;
    // check every layer before enqueueing anything [P2 四、"CSA2：三种模式"]
    bool have_index = false;
    for (int i = 0; i < n_layers; ++i) {
        const cskv_layer &L = layers[i];
        REQUIRE(L.mode == CSKV_MODE_FULL || L.mode == CSKV_MODE_REINDEX || L.mode == CSKV_MODE_REUSE,
                CSKV_EINVAL, "layer %d: unknown mode %d", i, L.mode);
        if ((rc = attn_args(cache, L.q, n_heads, L.idx, L.mode != CSKV_MODE_REUSE, k, L.swa, window, L.out,
                            L.lse, work, work_bytes)))
            return fail(rc, "layer %d: %s", i, g_error.c_str());
        REQUIRE(!L.swa_row || aligned(L.swa_row, 16), CSKV_EINVAL, "layer %d: swa_row not 16-byte aligned", i);
        if (L.mode == CSKV_MODE_REUSE) {
            REQUIRE(have_index, CSKV_EINVAL, "layer %d: REUSE with no FULL/REINDEX layer before it", i);
        } else {
            if ((rc = topk_args(cache, L.q_idx, n_idx_heads, k, L.idx, work, work_bytes)))
                return fail(rc, "layer %d: %s", i, g_error.c_str());
            have_index = true;
        }
    }
    return CSKV_OK;
}

// Enqueue one checked layer-group step.  The pool (if any) sits at the start
// of ws; each step uses what follows.
static int run_group(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                     const float *new_tokens, const float *w_comp, const uint16_t *new_idx_rows,
                     int32_t n_idx_heads, int32_t n_heads, int32_t k, int32_t window, float softmax_scale,
                     int32_t pool_blocks, int32_t pool_block, void *ws, size_t ws_bytes, hipStream_t stream)
{
    const size_t pool_bytes = group_pool_bytes(*cache, pool_blocks);
    int32_t *pool = pool_blocks > 0 ? static_cast<int32_t *>(ws) : nullptr;
    void *work = static_cast<char *>(ws) + pool_bytes;
    bool appended = false, pooled = false;
    const int32_t *last_idx = nullptr;
    // A compressor append rides on the first FULL layer's top-k when the
    // bound select serves the cache and the workspace holds the entry: the
    // head kernel advances the cache before the scan, the top-k's launches
    // compress and quantise the entry before attention reads it.
    const size_t carry_off = group_carry_off(*cache, k, pool_blocks, pool_block);
    const cskv::DeferredEntry carry =
        cskv::deferred_entry_at(static_cast<char *>(work) + carry_off, cache->batch, new_tokens, w_comp);
    const bool can_carry = w_comp && cskv::topk_carries_entry(*cache, k) &&
                           ws_bytes >= pool_bytes + carry_off + cskv::deferred_entry_bytes(cache->batch);
    const cskv::DeferredEntry *carried = nullptr;
    hipError_t e;
    for (int i = 0; i < n_layers; ++i) {
        const cskv_layer &L = layers[i];
        bool window_done = false;
        if (L.mode == CSKV_MODE_FULL && new_tokens && !appended) {
            // the append also writes this layer's window row
            if (can_carry) {
                e = cskv::launch_append_head(*cache, carry, new_idx_rows, stream, L.swa_row ? L.swa : nullptr,
                                             L.swa_row, window);
                carried = &carry;
            } else {
                e = cskv::launch_kv_append(*cache, new_tokens, nullptr, cache->batch, w_comp, new_idx_rows, work,
                                           stream, L.swa_row ? L.swa : nullptr, L.swa_row, window);
            }
            if (e != hipSuccess) return hip_fail(e, "layer group: append");
            appended = true;
            window_done = L.swa_row != nullptr;
        }
        if (L.swa_row && !window_done) {
            e = cskv::launch_swa_append(L.swa, cache->batch, window, cache->dim, L.swa_row, nullptr,
                                        cache->batch, cache->n_tokens, stream,
                                        cache->swa_format == CSKV_SWA_FP8);
            if (e != hipSuccess) return hip_fail(e, "layer group: window append");
        }
        if (L.mode == CSKV_MODE_REINDEX && pooled) {
            // hierarchical indexer: select inside the first FULL layer's pool
            e = cskv::launch_indexer_topk_in_pool(*cache, L.q_idx, n_idx_heads, L.head_w, k, pool, pool_blocks,
                                                  pool_block, L.idx, work, stream);
            if (e != hipSuccess) return hip_fail(e, "layer group: pooled indexer");
            last_idx = L.idx;
        } else if (L.mode != CSKV_MODE_REUSE) {
            const bool build = pool && L.mode == CSKV_MODE_FULL && !pooled;
            const cskv::PoolBuild pb{pool_blocks, pool_block, pool};
            e = cskv::launch_indexer_topk(*cache, L.q_idx, n_idx_heads, L.head_w, k, L.idx, work, stream,
                                          build ? &pb : nullptr, nullptr, carried);
            if (e != hipSuccess) return hip_fail(e, "layer group: indexer");
            carried = nullptr;
            pooled = pooled || build;
            last_idx = L.idx;
        }
        e = cskv::launch_sparse_attn(*cache, L.q, n_heads, last_idx, k, L.swa, window, nullptr,
                                     softmax_scale, L.out, L.lse, work, stream);
        if (e != hipSuccess) return hip_fail(e, "layer group: attention");
    }
    return CSKV_OK;
}

static int layer_group(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                       const float *new_tokens, const float *w_comp, const uint16_t *new_idx_rows,
                       int32_t n_idx_heads, int32_t n_heads, int32_t k, int32_t window,
                       float softmax_scale, int32_t pool_blocks, int32_t pool_block, void *ws,
                       size_t ws_bytes, hipStream_t stream)
{
    const int rc = check_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads,
                               k, window, pool_blocks, pool_block, ws, ws_bytes);
    if (rc) return rc;
    return run_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads, k, window,
                     softmax_scale, pool_blocks, pool_block, ws, ws_bytes, stream);
}

static int ced_args(const uint16_t *h, int64_t rows, int32_t d_model, const uint16_t *w, int32_t n_out,
                    const float *out)
{
    REQUIRE(rows >= 0 && rows <= (1 << 22), CSKV_EINVAL, "rows %lld out of [0, 2^22]", (long long)rows);
    REQUIRE(d_model >= 128 && d_model <= 65536 && d_model % 128 == 0, CSKV_EUNSUPPORTED,
            "d_model %d: a multiple of 128 in [128, 65536]", d_model);
    REQUIRE(n_out >= 16 && n_out <= 65536 && n_out % 16 == 0, CSKV_EUNSUPPORTED,
            "n_out %d: a multiple of 16 in [16, 65536]", n_out);
    REQUIRE(rows == 0 || (h && w && out), CSKV_EINVAL, "h, w or out is NULL");
    REQUIRE(aligned(h, 16) && aligned(w, 16) && aligned(out, 16), CSKV_EINVAL,
            "h, w and out must be 16-byte aligned");
    return CSKV_OK;
}

static size_t ced_rows_bytes(const cskv_cache &c) { return ((size_t)c.batch * c.dim * 4 + 255) / 256 * 256; }

int cskv_layer_group_decode(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                            const float *new_tokens, const float *w_comp,
                            const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                            int32_t k, int32_t window, float softmax_scale, void *ws,
                            size_t ws_bytes, hipStream_t stream)
{
    return layer_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads, k,
                       window, softmax_scale, 0, 0, ws, ws_bytes, stream);
}

int cskv_layer_group_decode_noalloc(const cskv_cache *cache, const cskv_layer *layers, int32_t n_layers,
                                    const float *new_tokens, const float *w_comp,
                                    const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                                    int32_t k, int32_t window, float softmax_scale, hipStream_t stream)
{
    int rc = check_cache(cache);
    if (rc) return rc;
    REQUIRE(n_heads >= 16 && n_heads <= 1024 && n_heads % 16 == 0 && k >= 1 && k <= 2048 && window >= 1 &&
                window <= 1024,
            CSKV_EUNSUPPORTED, "n_heads %d, k %d or window %d outside the supported range", n_heads, k, window);
    const size_t need = group_ws_bytes(*cache, n_heads, k, window, 0, 0);
    REQUIRE(need <= (size_t)CSKV_NOALLOC_SCRATCH_BYTES, CSKV_EWORKSPACE,
            "this step needs %zu bytes of workspace; the built-in scratch holds %zu "
            "(use cskv_layer_group_decode with a caller workspace)",
            need, (size_t)CSKV_NOALLOC_SCRATCH_BYTES);
    // every argument is checked before the scratch is looked up (the check
    // reads only the workspace's size and alignment, not its address)
    void *const placeholder = reinterpret_cast<void *>((uintptr_t)256);
    if ((rc = check_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads, k,
                          window, 0, 0, placeholder, (size_t)CSKV_NOALLOC_SCRATCH_BYTES)))
        return rc;
    void *ws = nullptr;
    if ((rc = scratch_of_current_device(&ws))) return rc;
    return run_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads, k, window,
                     softmax_scale, 0, 0, ws, (size_t)CSKV_NOALLOC_SCRATCH_BYTES, stream);
}

int cskv_layer_group_decode_pooled(const cskv_cache *cache, const cskv_layer *layers,
                                   int32_t n_layers, const float *new_tokens, const float *w_comp,
                                   const uint16_t *new_idx_rows, int32_t n_idx_heads, int32_t n_heads,
                                   int32_t k, int32_t window, float softmax_scale, int32_t pool_blocks,
                                   int32_t pool_block, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return layer_group(cache, layers, n_layers, new_tokens, w_comp, new_idx_rows, n_idx_heads, n_heads, k,
                       window, softmax_scale, pool_blocks, pool_block, ws, ws_bytes, stream);
}

int cskv_ced_project(const uint16_t *h, int64_t rows, int32_t d_model, const uint16_t *w, int32_t n_out,
                     float *out, hipStream_t stream)
{
    const int rc = ced_args(h, rows, d_model, w, n_out, out);
    if (rc) return rc;
    const hipError_t e = cskv::launch_ced_project(h, rows, d_model, w, n_out, out, stream);
    return e == hipSuccess ? CSKV_OK : hip_fail(e, "ced_project launch");
}

// Per group: the workspace its layer group needs after the CED rows.
static size_t model_ws_bytes(const cskv_group *groups, int32_t n_groups, int32_t n_heads, int32_t k,
                             int32_t window)
{
    size_t rows = 0, group = 0;
    for (int g = 0; g < n_groups; ++g) {
        const cskv_cache &c = *groups[g].cache;
        if (groups[g].ced_h) rows = std::max(rows, ced_rows_bytes(c));
        group = std::max(group, group_ws_bytes(c, n_heads, k, window, groups[g].pool_blocks, groups[g].pool_block));
    }
    return rows + group;
}

static int check_model(const cskv_group *groups, int32_t n_groups, int32_t n_heads, int32_t k, int32_t window)
{
    REQUIRE(groups && n_groups >= 1 && n_groups <= 64, CSKV_EINVAL, "need 1..64 groups");
    for (int g = 0; g < n_groups; ++g) {
        const cskv_group &G = groups[g];
        int rc = check_cache(G.cache);
        if (rc) return fail(rc, "group %d: %s", g, g_error.c_str());
        REQUIRE(!(G.new_tokens && G.ced_h), CSKV_EINVAL, "group %d: new_tokens and ced_h are exclusive", g);
        if (G.ced_h) {
            REQUIRE(G.new_idx_rows, CSKV_EINVAL, "group %d: ced_h needs new_idx_rows", g);
            float *dummy = reinterpret_cast<float *>(256);      // alignment-only stand-in for the rows
            if ((rc = ced_args(G.ced_h, G.cache->batch, G.d_model, G.ced_w, G.cache->dim, dummy)))
                return fail(rc, "group %d: %s", g, g_error.c_str());
        }
        if (G.pool_blocks != 0 && (rc = pool_args(G.cache, k, G.pool_blocks, G.pool_block)))
            return fail(rc, "group %d: %s", g, g_error.c_str());
    }
    (void)n_heads;
    (void)window;
    return CSKV_OK;
}

size_t cskv_model_workspace_bytes(const cskv_group *groups, int32_t n_groups, int32_t n_heads, int32_t k,
                                  int32_t window)
{
    if (check_model(groups, n_groups, n_heads, k, window) != CSKV_OK) return 0;
    return model_ws_bytes(groups, n_groups, n_heads, k, window);
}

int cskv_model_decode(const cskv_group *groups, int32_t n_groups, int32_t n_idx_heads, int32_t n_heads,
                      int32_t k, int32_t window, float softmax_scale, void *ws, size_t ws_bytes,
                      hipStream_t stream)
{
    int rc = check_model(groups, n_groups, n_heads, k, window);
    if (rc) return rc;
    REQUIRE(ws && aligned(ws, 256), CSKV_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    const size_t need = model_ws_bytes(groups, n_groups, n_heads, k, window);
    REQUIRE(ws_bytes >= need, CSKV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    size_t rows_bytes = 0;
    for (int g = 0; g < n_groups; ++g)
        if (groups[g].ced_h) rows_bytes = std::max(rows_bytes, ced_rows_bytes(*groups[g].cache));
    float *rows = reinterpret_cast<float *>(ws);
    void *gws = static_cast<char *>(ws) + rows_bytes;
    const size_t gws_bytes = ws_bytes - rows_bytes;
    // every group is checked before anything is enqueued
    for (int g = 0; g < n_groups; ++g) {
        const cskv_group &G = groups[g];
        const float *src = G.ced_h ? rows : G.new_tokens;
        if ((rc = check_group(G.cache, G.layers, G.n_layers, src, G.ced_h ? nullptr : G.w_comp, G.new_idx_rows,
                              n_idx_heads, n_heads, k, window, G.pool_blocks, G.pool_block, gws, gws_bytes)))
            return fail(rc, "group %d: %s", g, g_error.c_str());
    }
    for (int g = 0; g < n_groups; ++g) {
        const cskv_group &G = groups[g];
        if (G.ced_h) {
            const hipError_t e = cskv::launch_ced_project(G.ced_h, G.cache->batch, G.d_model, G.ced_w,
                                                          G.cache->dim, rows, stream);
            if (e != hipSuccess) return hip_fail(e, "model decode: CED projection");
        }
        if ((rc = run_group(G.cache, G.layers, G.n_layers, G.ced_h ? rows : G.new_tokens,
                            G.ced_h ? nullptr : G.w_comp, G.new_idx_rows, n_idx_heads, n_heads, k, window,
                            softmax_scale, G.pool_blocks, G.pool_block, gws, gws_bytes, stream)))
            return rc;
    }
    return CSKV_OK;
}

int cskv_timer_enable(int32_t kind, int32_t max_launches)
{
    REQUIRE(kind >= 1 && kind < 8, CSKV_EINVAL, "kernel kind %d", kind);
    REQUIRE(max_launches >= 1 && max_launches <= 1 << 16, CSKV_EINVAL, "max_launches %d", max_launches);
    Timer &T = g_timers[kind];
    free_timer(T);
    T.start.resize(max_launches);
    T.stop.resize(max_launches);
    for (int i = 0; i < max_launches; ++i) {
        hipError_t e1 = hipEventCreate(&T.start[i]), e2 = hipEventCreate(&T.stop[i]);
        if (e1 != hipSuccess || e2 != hipSuccess) {
            free_timer(T);
            return hip_fail(e1 != hipSuccess ? e1 : e2, "hipEventCreate");
        }
    }
    T.max = max_launches;
    T.on = true;
    return CSKV_OK;
}

int cskv_timer_pause(int32_t kind, int32_t paused)
{
    REQUIRE(kind >= 1 && kind < 8, CSKV_EINVAL, "kernel kind %d", kind);
    g_timers[kind].paused = paused != 0;
    return CSKV_OK;
}

int cskv_timer_read(int32_t kind, double *total_ms, int32_t *count)
{
    REQUIRE(kind >= 1 && kind < 8 && total_ms && count, CSKV_EINVAL, "bad timer_read arguments");
    Timer &T = g_timers[kind];
    double sum = 0;
    for (int i = 0; i < T.count; ++i) {
        hipError_t e = hipEventSynchronize(T.stop[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0;
        e = hipEventElapsedTime(&ms, T.start[i], T.stop[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        sum += ms;
    }
    *total_ms = sum;
    *count = T.count;
    return CSKV_OK;
}

int cskv_timer_disable_all(void)
{
    for (auto &T : g_timers) free_timer(T);
    return CSKV_OK;
}

}  // extern "C"
