// append.hip -- cache append: 2->1 compression, group FP4 quantisation and
// packing, pending-token bookkeeping, and the sliding-window rows.
//
// Sources cited as [P1]/[P2] (page title, then the section):
//   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {
namespace {

constexpr int kDim = 576;          // entry dims handled by these kernels (512 latent + 64 RoPE)
constexpr int kAppendThreads = kDim;  // one channel per thread, 9 waves

struct AppendArgs {
    cskv_cache c;
    const float *tokens;
    const int32_t *cu_new;
    const float *w_comp;
    const uint16_t *idx_rows;
    int64_t total_new;
};

// Rows of sequence b are [row0, row0 + m).  A malformed cu_new (decreasing,
// or pointing past total_new) must not make any row be read or written out of
// bounds: such a sequence is rejected as a whole.
__device__ __forceinline__ bool rows_ok(int64_t row0, int64_t m, int64_t total)
{
    return row0 >= 0 && m >= 0 && row0 + m <= total;
}

// Group absmax of the channel each thread holds (threads >= n hold 0).
// Groups of g <= 64 channels lie inside one wave and reduce with lane
// exchanges; g = 128 adds one combine of two wave results through LDS.
__device__ float group_absmax(float a, int t, int n, int g, float *wave_max)
{
    const int span = g < kWave ? g : kWave;
    for (int off = span >> 1; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if (g > kWave) {
        if ((t & (kWave - 1)) == 0) wave_max[t / kWave] = a;
        __syncthreads();
        const int per = g / kWave, first = (t / g) * per;
        float m = 0.f;
        if (t < n)                                  // groups of live channels only
            for (int i = 0; i < per; ++i) m = fmaxf(m, wave_max[first + i]);
        __syncthreads();
        a = m;
    }
    return a;
}

// Quantise channel t of a row of n channels with group g into a packed plane
// row [P1 §3.1 (per-group scale, values stored relative to it); P2 四、"P4 main
// KV" (E2M1)].  Called by all threads of the block (it contains barriers).
__device__ void quantize_channel(float x, int t, int n, int g, uint8_t *codes_row,
                                 float *scales_row, float *wave_max)
{
    const bool live = t < n;
    float a = group_absmax(live ? fabsf(x) : 0.f, t, n, g, wave_max);
    const float s = a / 6.0f;                      // IEEE division (no fast-math)
    uint32_t code = (live && s != 0.0f) ? e2m1_code(x / s) : 0u;
    uint32_t hi = __shfl_down(code, 1);
    if (live && (t & 1) == 0) codes_row[t >> 1] = (uint8_t)(code | (hi << 4));
    if (live && (t % g) == 0) scales_row[t / g] = s;
}

// One block per input row.  A block whose row completes an entry (compressor
// mode: the row sits at an odd absolute position; entries mode: every row)
// computes that entry and writes its codes, scales and indexer key.
template <bool kCompress>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a)
{
    __shared__ float u[2 * kDim];
    __shared__ float wave_max[kAppendThreads / kWave];
    const cskv_cache &c = a.c;
    const int r = blockIdx.x, t = threadIdx.x;
    const int b = seq_of_row(a.cu_new, c.batch, r);
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    const int64_t q = r - row0;
    const int64_t p = c.n_tokens[b];
    if (p < 0 || !rows_ok(row0, m, a.total_new) || q < 0 || q >= m) return;
    int64_t entry;
    if (kCompress) {
        const int64_t pos = p + q;
        if ((pos & 1) == 0) return;                    // first half of a pair
        if ((p + m) / 2 > c.capacity) return;          // rejected sequence (finalize flags it)
        entry = pos >> 1;
    } else {
        if ((p & 1) != 0 || p / 2 + m > c.capacity) return;
        entry = p / 2 + q;
    }

    float e;
    if (kCompress) {
        // Stand-in compressor: e[t] = sum_j W[t][j] u[j], u = x_even || x_odd,
        // one fused multiply-add per term in increasing j.
        const float *x_even = (q > 0) ? a.tokens + (size_t)(r - 1) * kDim
                                      : c.pending + (size_t)b * kDim;
        u[t] = x_even[t];
        u[kDim + t] = a.tokens[(size_t)r * kDim + t];
        __syncthreads();
        const float4 *wrow = reinterpret_cast<const float4 *>(a.w_comp + (size_t)t * 2 * kDim);
        float acc = 0.0f;
#pragma unroll 4
        for (int j4 = 0; j4 < 2 * kDim / 4; ++j4) {
            const float4 w = wrow[j4];
            acc = fmaf(w.x, u[4 * j4 + 0], acc);
            acc = fmaf(w.y, u[4 * j4 + 1], acc);
            acc = fmaf(w.z, u[4 * j4 + 2], acc);
            acc = fmaf(w.w, u[4 * j4 + 3], acc);
        }
        e = acc;
    } else {
        e = a.tokens[(size_t)r * kDim + t];
    }

    const size_t slot = (size_t)b * c.capacity + (size_t)entry;
    quantize_channel(e, t, kDim, c.k_group, c.k_codes + slot * (kDim / 2),
                     c.k_scales + slot * (kDim / c.k_group), wave_max);
    if (c.v_group > 0) {
        const int dv = c.dim - c.rope_dim;
        quantize_channel(e, t, dv, c.v_group, c.v_codes + slot * (dv / 2),
                         c.v_scales + slot * (dv / c.v_group), wave_max);
    }
    if (t < c.idx_dim) c.idx_keys[slot * c.idx_dim + t] = a.idx_rows[(size_t)r * c.idx_dim + t];
}

// One wave per sequence, after append_kernel: stores the trailing odd token,
// advances n_tokens, or flags a rejected sequence.
template <bool kCompress>
__global__ __launch_bounds__(kWave) void append_finalize_kernel(AppendArgs a)
{
    const cskv_cache &c = a.c;
    const int b = blockIdx.x, t = threadIdx.x;
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    const int64_t p = c.n_tokens[b];
    if (m == 0) return;
    if (p < 0 || !rows_ok(row0, m, a.total_new)) {
        if (t == 0) atomicOr(c.status, CSKV_STATUS_BAD_STATE);
        return;
    }
    if (kCompress) {
        if ((p + m) / 2 > c.capacity) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_OVERFLOW);
            return;
        }
        if (((p + m) & 1) != 0) {
            const float *last = a.tokens + (size_t)(row0 + m - 1) * kDim;
            for (int i = t; i < kDim; i += kWave) c.pending[(size_t)b * kDim + i] = last[i];
        }
        if (t == 0) c.n_tokens[b] = (int32_t)(p + m);
    } else {
        if ((p & 1) != 0) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_ODD_ENTRY_APPEND);
            return;
        }
        if (p / 2 + m > c.capacity) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_OVERFLOW);
            return;
        }
        if (t == 0) c.n_tokens[b] = (int32_t)(p + 2 * m);
    }
}

struct SwaArgs {
    uint16_t *ring;
    int batch, window, dim;
    const float *rows;
    const int32_t *cu_new;
    const int32_t *end_pos;
    int64_t total_new;
};

// One wave per row: fp32 -> bf16 (nearest even) into ring slot pos % window
// when the row is among the last `window` positions.
__global__ __launch_bounds__(kWave) void swa_append_kernel(SwaArgs a)
{
    const int r = blockIdx.x, t = threadIdx.x;
    const int b = seq_of_row(a.cu_new, a.batch, r);
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    const int64_t end = a.end_pos[b];
    const int64_t pos = end - m + (r - row0);
    if (!rows_ok(row0, m, a.total_new) || r - row0 >= m) return;
    if (pos < 0 || pos < end - a.window) return;
    const float4 *src = reinterpret_cast<const float4 *>(a.rows + (size_t)r * a.dim);
    uint2 *dst = reinterpret_cast<uint2 *>(a.ring + ((size_t)b * a.window + (size_t)(pos % a.window)) * a.dim);
    for (int i = t; i < a.dim / 4; i += kWave) {
        const float4 x = src[i];
        uint2 o;
        o.x = bf16_bits_rne(x.x) | (bf16_bits_rne(x.y) << 16);
        o.y = bf16_bits_rne(x.z) | (bf16_bits_rne(x.w) << 16);
        dst[i] = o;
    }
}

}  // namespace

hipError_t launch_kv_append(const cskv_cache &c, const float *tokens, const int32_t *cu_new,
                            int total_new, const float *w_comp, const uint16_t *idx_rows,
                            hipStream_t s)
{
    if (total_new == 0) return hipSuccess;
    AppendArgs a{c, tokens, cu_new, w_comp, idx_rows, total_new};
    timer_before(CSKV_KERNEL_APPEND, s);
    if (w_comp) {
        append_kernel<true><<<total_new, kAppendThreads, 0, s>>>(a);
        append_finalize_kernel<true><<<c.batch, kWave, 0, s>>>(a);
    } else {
        append_kernel<false><<<total_new, kAppendThreads, 0, s>>>(a);
        append_finalize_kernel<false><<<c.batch, kWave, 0, s>>>(a);
    }
    timer_after(CSKV_KERNEL_APPEND, s);
    return hipGetLastError();
}

hipError_t launch_swa_append(uint16_t *ring, int batch, int window, int dim, const float *rows,
                             const int32_t *cu_new, int total_new, const int32_t *end_pos,
                             hipStream_t s)
{
    if (total_new == 0) return hipSuccess;
    SwaArgs a{ring, batch, window, dim, rows, cu_new, end_pos, total_new};
    timer_before(CSKV_KERNEL_SWA_APPEND, s);
    swa_append_kernel<<<total_new, kWave, 0, s>>>(a);
    timer_after(CSKV_KERNEL_SWA_APPEND, s);
    return hipGetLastError();
}

}  // namespace cskv
