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
constexpr int kAppendThreads = kDim;  // quantiser: one channel per thread, 9 waves

struct AppendArgs {
    cskv_cache c;
    const float *tokens;
    const int32_t *cu_new;
    const float *w_comp;
    const uint16_t *idx_rows;
    float *ent;          // compressor output, [total_new][dim] (rows that complete an entry)
    int64_t total_new;
};

// Rows of sequence b are [row0, row0 + m).  A malformed cu_new (decreasing,
// or pointing past total_new) must not make any row be read or written out of
// bounds: such a sequence is rejected as a whole.
__device__ __forceinline__ bool rows_ok(int64_t row0, int64_t m, int64_t total)
{
    return row0 >= 0 && m >= 0 && row0 + m <= total;
}

// Where input row r lands: the cache slot of the entry it completes, or -1
// when it completes none (first half of a pair, a rejected sequence, a bad
// row).  Also the sequence and the row of its pair partner (-1: pending).
struct RowInfo {
    int b;
    int64_t entry;       // entry index within the sequence, or -1
    int64_t partner;     // compressor mode: input row of x_even, -1 = pending[b]
};

template <bool kCompress>
__device__ __forceinline__ RowInfo row_info(const AppendArgs &a, int64_t r)
{
    const cskv_cache &c = a.c;
    RowInfo ri{0, -1, -1};
    const int b = seq_of_row(a.cu_new, c.batch, (int)r);
    ri.b = b;
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    const int64_t q = r - row0;
    const int64_t p = c.n_tokens[b];
    if (p < 0 || !rows_ok(row0, m, a.total_new) || q < 0 || q >= m) return ri;
    if (kCompress) {
        const int64_t pos = p + q;
        if ((pos & 1) == 0) return ri;                 // first half of a pair
        if ((p + m) / 2 > c.capacity) return ri;       // rejected sequence (finalize flags it)
        ri.entry = pos >> 1;
        ri.partner = q > 0 ? r - 1 : -1;
    } else {
        if ((p & 1) != 0 || p / 2 + m > c.capacity) return ri;
        ri.entry = p / 2 + q;
    }
    return ri;
}

// ---------------------------------------------------------------- compressor

// Stand-in 2->1 compressor [P2 三、"突破四" (2 tokens -> 1 entry); P1 §3.2]:
// e[ch] = sum_j W[ch][j] u[j], u = x_even || x_odd, folded in fp32 from j = 0
// upward with one fused multiply-add per term.  Each output channel is one
// sequential chain of 2*dim dependent FMAs, so the parallelism is channels x
// entries: one wave takes 64 channels (one per lane) of NE consecutive input
// rows, reads its W rows once for all of them and keeps one accumulator per
// row.  The rows' inputs u are staged in LDS and read as broadcasts.
template <int NE>
__global__ __launch_bounds__(kWave) void compress_kernel(AppendArgs a)
{
    __shared__ float4 u_s[NE][2 * kDim / 4];
    __shared__ const float *src_s[NE][2];
    const int lane = threadIdx.x, rb = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * NE;

    bool act = false;
    if (lane < NE && r0 + lane < a.total_new) {
        const int64_t r = r0 + lane;
        const RowInfo ri = row_info<true>(a, r);
        if (ri.entry >= 0) {
            act = true;
            src_s[lane][0] = ri.partner >= 0 ? a.tokens + (size_t)ri.partner * kDim
                                             : a.c.pending + (size_t)ri.b * kDim;
            src_s[lane][1] = a.tokens + (size_t)r * kDim;
        }
    }
    const uint64_t am = __ballot(act);
    if (am == 0) return;
    __syncthreads();

    // stage u of every active row: 2 x 144 float4 per row
#pragma unroll 1
    for (int e = 0; e < NE; ++e) {
        if (!((am >> e) & 1ull)) continue;
        const float4 *xe = reinterpret_cast<const float4 *>(src_s[e][0]);
        const float4 *xo = reinterpret_cast<const float4 *>(src_s[e][1]);
        for (int i = lane; i < kDim / 4; i += kWave) {
            u_s[e][i] = xe[i];
            u_s[e][kDim / 4 + i] = xo[i];
        }
    }
    __syncthreads();

    const int ch = kWave * rb + lane;
    const float4 *wrow = reinterpret_cast<const float4 *>(a.w_comp + (size_t)ch * 2 * kDim);
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
    constexpr int kQ = 2 * kDim / 4;       // 288 float4 per W row
    constexpr int kU = 8;                  // float4 per step
    float4 wcur[kU], wnext[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) wcur[i] = wrow[i];
    for (int j0 = 0; j0 < kQ; j0 += kU) {
        if (j0 + kU < kQ) {
#pragma unroll
            for (int i = 0; i < kU; ++i) wnext[i] = wrow[j0 + kU + i];
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if ((am >> e) & 1ull) {
                float x = acc[e];
#pragma unroll
                for (int i = 0; i < kU; ++i) {
                    const float4 u = u_s[e][j0 + i];
                    x = fmaf(wcur[i].x, u.x, x);
                    x = fmaf(wcur[i].y, u.y, x);
                    x = fmaf(wcur[i].z, u.z, x);
                    x = fmaf(wcur[i].w, u.w, x);
                }
                acc[e] = x;
            }
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) wcur[i] = wnext[i];
    }
#pragma unroll
    for (int e = 0; e < NE; ++e)
        if ((am >> e) & 1ull) a.ent[(size_t)(r0 + e) * kDim + ch] = acc[e];
}

// ---------------------------------------------------------------- quantiser

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
// KV" (E2M1)].  Codes are gathered 8 per 32-bit word with lane exchanges so
// that every eighth thread writes one word.  Called by all threads of the
// block (it contains barriers).
__device__ void quantize_channel(float x, int t, int n, int g, uint8_t *codes_row,
                                 float *scales_row, float *wave_max)
{
    const bool live = t < n;
    float a = group_absmax(live ? fabsf(x) : 0.f, t, n, g, wave_max);
    const float s = a / 6.0f;                      // IEEE division (no fast-math)
    uint32_t code = (live && s != 0.0f) ? e2m1_code(x / s) : 0u;
    code |= __shfl_down(code, 1) << 4;             // 2 codes (even t)
    code |= __shfl_down(code, 2) << 8;             // 4 codes (t % 4 == 0)
    code |= __shfl_down(code, 4) << 16;            // 8 codes (t % 8 == 0)
    if (live && (t & 7) == 0) *reinterpret_cast<uint32_t *>(codes_row + (t >> 1)) = code;
    if (live && (t % g) == 0) scales_row[t / g] = s;
}

// One block per input row.  A block whose row completes an entry quantises
// that entry (compressor mode: from the compressor's output; entries mode:
// the row itself) and writes its codes, scales and indexer key.
template <bool kCompress>
__global__ __launch_bounds__(kAppendThreads) void quantize_kernel(AppendArgs a)
{
    __shared__ float wave_max[kAppendThreads / kWave];
    const cskv_cache &c = a.c;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const RowInfo ri = row_info<kCompress>(a, r);
    if (ri.entry < 0) return;
    const float e = kCompress ? a.ent[(size_t)r * kDim + t] : a.tokens[(size_t)r * kDim + t];
    const size_t slot = (size_t)ri.b * c.capacity + (size_t)ri.entry;
    quantize_channel(e, t, kDim, c.k_group, c.k_codes + slot * (kDim / 2),
                     c.k_scales + slot * (kDim / c.k_group), wave_max);
    if (c.v_group > 0) {
        const int dv = c.dim - c.rope_dim;
        quantize_channel(e, t, dv, c.v_group, c.v_codes + slot * (dv / 2),
                         c.v_scales + slot * (dv / c.v_group), wave_max);
    }
    if (t < c.idx_dim) c.idx_keys[slot * c.idx_dim + t] = a.idx_rows[(size_t)r * c.idx_dim + t];
}

// One wave per sequence, after the quantiser: stores the trailing odd token,
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

size_t append_workspace_bytes(int total_new)
{
    return (size_t)total_new * kDim * sizeof(float);
}

hipError_t launch_kv_append(const cskv_cache &c, const float *tokens, const int32_t *cu_new,
                            int total_new, const float *w_comp, const uint16_t *idx_rows,
                            void *ws, hipStream_t s)
{
    if (total_new == 0) return hipSuccess;
    AppendArgs a{c, tokens, cu_new, w_comp, idx_rows, static_cast<float *>(ws), total_new};
    const TimedLaunch tl = timer_take(CSKV_KERNEL_APPEND);
    if (w_comp) {
        // decode-sized appends: one row per wave (shortest chains); large
        // chunks: 8 rows per wave share each W row read
        if (total_new <= 1024)
            launch_kernel(compress_kernel<1>, dim3((unsigned)total_new, kDim / kWave), dim3(kWave), s, tl.start,
                          nullptr, a);
        else
            launch_kernel(compress_kernel<8>, dim3((unsigned)((total_new + 7) / 8), kDim / kWave), dim3(kWave), s,
                          tl.start, nullptr, a);
        launch_kernel(quantize_kernel<true>, dim3((unsigned)total_new), dim3(kAppendThreads), s, nullptr, nullptr, a);
        launch_kernel(append_finalize_kernel<true>, dim3((unsigned)c.batch), dim3(kWave), s, nullptr, tl.stop, a);
    } else {
        launch_kernel(quantize_kernel<false>, dim3((unsigned)total_new), dim3(kAppendThreads), s, tl.start, nullptr,
                      a);
        launch_kernel(append_finalize_kernel<false>, dim3((unsigned)c.batch), dim3(kWave), s, nullptr, tl.stop, a);
    }
    return hipGetLastError();
}

hipError_t launch_swa_append(uint16_t *ring, int batch, int window, int dim, const float *rows,
                             const int32_t *cu_new, int total_new, const int32_t *end_pos,
                             hipStream_t s)
{
    if (total_new == 0) return hipSuccess;
    SwaArgs a{ring, batch, window, dim, rows, cu_new, end_pos, total_new};
    const TimedLaunch tl = timer_take(CSKV_KERNEL_SWA_APPEND);
    launch_kernel(swa_append_kernel, dim3((unsigned)total_new), dim3(kWave), s, tl.start, tl.stop, a);
    return hipGetLastError();
}

}  // namespace cskv
