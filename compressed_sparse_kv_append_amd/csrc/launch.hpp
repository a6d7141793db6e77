// launch.hpp -- host-side launchers of the kernels (internal to the library).
// Each returns hipSuccess or the launch error; argument checking happens in
// api.cpp before any of these is called.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cskv.h"

namespace cskv {

// Workspace layout of the indexer + top-k (offsets in bytes from ws): one
// uint32 score key per entry, and the per-slice candidate lists of sequences
// longer than one select round; or, for caches the tile select serves, the
// largest key of every 16-entry tile and one candidate list per sequence.
struct TopkWorkspace {
    size_t keys_off, cand_off, cand2_off, total;
    bool tiles = false;
    size_t tmax_off = 0, tmax_stride = 0, tcand_off = 0;
};
constexpr int kSliceKeys = 4096;  // keys per select slice (one block)
// Score keys: one uint32 per cache row; a sequence's rows padded to 64.
inline size_t score_key_stride(const cskv_cache &c) { return ((size_t)c.capacity + 63) / 64 * 64; }
TopkWorkspace topk_workspace(const cskv_cache &c, int k);
int topk_slices(const cskv_cache &c);

// Compressor output rows (fp32) staged between the compressor and the quantiser.
size_t append_workspace_bytes(int total_new);
// With cu_new == nullptr (one row per sequence) the quantiser also finalises
// each sequence and, when swa_ring is given, writes swa_rows[b] into that
// ring at the row's token position (what launch_swa_append would do).
hipError_t launch_kv_append(const cskv_cache &c, const float *tokens, const int32_t *cu_new,
                            int total_new, const float *w_comp, const uint16_t *idx_rows,
                            void *ws, hipStream_t s, uint16_t *swa_ring = nullptr,
                            const float *swa_rows = nullptr, int swa_window = 0, bool mfma = false);
// fp8: the ring holds E4M3 bytes (dim a multiple of 16), else bf16 (dim a
// multiple of 4).
hipError_t launch_ced_project(const uint16_t *h, int64_t rows, int d_model, const uint16_t *w, int n_out,
                              float *out, hipStream_t s);
hipError_t launch_swa_append(uint16_t *ring, int batch, int window, int dim, const float *rows,
                             const int32_t *cu_new, int total_new, const int32_t *end_pos,
                             hipStream_t s, bool fp8 = false);
// Indexer scan (scan.hip): one score key per valid entry into keys
// [batch][score_key_stride]; with block_keys, also the largest key of each
// block of `block` entries (block divides 16) into block_keys
// [batch][block_stride]; with out_scores, the fp32 score of every live
// entry into out_scores [batch][capacity].
void launch_indexer_scan(const cskv_cache &c, const uint16_t *q_idx, int heads, const float *head_w,
                         uint32_t *keys, hipStream_t s, uint32_t *block_keys = nullptr,
                         size_t block_stride = 0, int block = 1, float *out_scores = nullptr,
                         uint32_t *tile_max = nullptr, size_t tile_stride = 0);
// Pooled scan (scan.hip): (score key, entry) pairs of the entries of the
// pooled blocks, pairs [batch][pool_blocks * block] in pool order; key 0 and
// entry ~0 where a position holds no entry.
void launch_pool_scan(const cskv_cache &c, const uint16_t *q_idx, int heads, const float *head_w,
                      const int32_t *pool, int pool_blocks, int block, uint2 *pairs, hipStream_t s);
// Candidate pool of the hierarchical indexer, built from the same scan as a
// layer's top-k: the best `blocks` blocks of `block` entries by their best
// score, ascending block indices into out [batch][blocks], -1 padded.
struct PoolBuild {
    int blocks, block;
    int32_t *out;
};
// Workspace of the pool: block keys and the block select's candidate lists
// after the top-k's own region (build_total in all), or the pooled scan's
// (key, entry) pairs from offset 0 (inpool_total).
struct PoolWorkspace {
    size_t bkeys_off, bkey_stride, bcand_off, bcand_stride, build_total, inpool_total;
    int bslices;
};
PoolWorkspace pool_workspace(const cskv_cache &c, int k, int pool_blocks, int block);
// A decode step's append (one new token per sequence, compressor mode)
// spread over the step's first top-k: launch_append_head writes each
// completed entry's indexer key, the pending tokens, the token counts and
// the window row, and records the new entry's cache row in slots (-1: none);
// launch_indexer_topk with `entry` then compresses the entry in its slice
// launch and quantises it into the cache in its final launch, so attention,
// which follows, reads it.  Only the bound select carries an entry, for at
// most 64 sequences (topk_carries_entry).  ent and slots live beside the top-k's workspace
// (deferred_entry_bytes).
struct DeferredEntry {
    const float *tokens;   // [batch][576] the step's tokens
    const float *w_comp;   // [576][1152] compressor weights
    float *ent;            // [batch][576] the compressor's output
    int64_t *slots;        // [batch] the cache row of each new entry, -1: none
};
size_t deferred_entry_bytes(int batch);
// ent and slots laid out from base (256-byte aligned, deferred_entry_bytes long).
DeferredEntry deferred_entry_at(void *base, int batch, const float *tokens, const float *w_comp);
hipError_t launch_append_head(const cskv_cache &c, const DeferredEntry &d, const uint16_t *idx_rows,
                              hipStream_t s, uint16_t *swa_ring, const float *swa_rows, int swa_window);
bool topk_carries_entry(const cskv_cache &c, int k);
hipError_t launch_indexer_topk(const cskv_cache &c, const uint16_t *q_idx, int heads,
                               const float *head_w, int k, int32_t *out_idx, void *ws,
                               hipStream_t s, const PoolBuild *pool = nullptr, float *out_scores = nullptr,
                               const DeferredEntry *entry = nullptr);
// Top-k among the entries of the pooled blocks (a later layer of the
// hierarchical indexer); ws holds pool_workspace().inpool_total bytes.
hipError_t launch_indexer_topk_in_pool(const cskv_cache &c, const uint16_t *q_idx, int heads,
                                       const float *head_w, int k, const int32_t *pool, int pool_blocks,
                                       int block, int32_t *out_idx, void *ws, hipStream_t s);
// Split of the keys of one (sequence, head group) over blocks: selected
// entries in chunks of 128, window rows in chunks of 64.  Split i takes entry
// chunks [i per_sparse, (i + 1) per_sparse) and window chunks
// [(i - win_split0) per_win, (i - win_split0 + 1) per_win), each clipped to
// what exists (none for i < win_split0).  win_split0 = 0 mixes both kinds in
// one split; win_split0 = the number of entry splits keeps each split to one
// kind.  ws_bytes: partial results when splits > 1.
struct AttnPlan {
    int n_sparse, n_win;
    int win_split0, per_sparse, per_win, splits;
    size_t ws_bytes;
};
AttnPlan attn_plan(const cskv_cache &c, int heads, int k, int window);
hipError_t launch_sparse_attn(const cskv_cache &c, const float *q, int heads, const int32_t *idx,
                              int k, const uint16_t *swa, int window, const int32_t *swa_len,
                              float scale, float *out, float *lse, void *ws, hipStream_t s);

// Kernel timers (api.cpp).  When the timer of a kernel kind is on, one
// launch group of that kind takes an event pair: its first kernel records
// `start` as it begins and its last records `stop` as it ends (both through
// hipExtLaunchKernel), so the interval covers the kernels' own execution and
// adds no marker packets to the stream.  Both are null when the timer is off.
struct TimedLaunch {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimedLaunch timer_take(int kind);

template <class... P, class... A>
inline void launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                          hipEvent_t stop, A... args)
{
    if (start || stop) hipExtLaunchKernelGGL(k, grid, block, 0, s, start, stop, 0, args...);
    else hipLaunchKernelGGL(k, grid, block, 0, s, args...);
}

}  // namespace cskv
