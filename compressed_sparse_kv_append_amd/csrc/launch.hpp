// launch.hpp -- host-side launchers of the kernels (internal to the library).
// Each returns hipSuccess or the launch error; argument checking happens in
// api.cpp before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cskv.h"

namespace cskv {

// Workspace layout of the indexer + top-k (offsets in bytes from ws).
struct TopkWorkspace {
    size_t keys_off, hist_off, total;
};
constexpr int kHistBins = 2048;   // first radix pass: top 11 bits of the key
TopkWorkspace topk_workspace(const cskv_cache &c);

hipError_t launch_kv_append(const cskv_cache &c, const float *tokens, const int32_t *cu_new,
                            int total_new, const float *w_comp, const uint16_t *idx_rows,
                            hipStream_t s);
hipError_t launch_swa_append(uint16_t *ring, int batch, int window, int dim, const float *rows,
                             const int32_t *cu_new, int total_new, const int32_t *end_pos,
                             hipStream_t s);
hipError_t launch_indexer_topk(const cskv_cache &c, const uint16_t *q_idx, int heads,
                               const float *head_w, int k, int32_t *out_idx, void *ws,
                               hipStream_t s);
hipError_t launch_sparse_attn(const cskv_cache &c, const float *q, int heads, const int32_t *idx,
                              int k, const uint16_t *swa, int window, const int32_t *swa_len,
                              float scale, float *out, float *lse, hipStream_t s);

// Kernel timers (api.cpp): bracket a launch with event records when enabled.
void timer_before(int kind, hipStream_t s);
void timer_after(int kind, hipStream_t s);

}  // namespace cskv
