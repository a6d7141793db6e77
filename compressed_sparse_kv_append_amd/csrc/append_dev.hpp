// append_dev.hpp -- device code of the cache append shared by its own
// kernels and by the top-k launches that carry a decode step's deferred
// entry: 2->1 compression, group FP4 quantisation and packing, the FP4
// indexer key, pending-token bookkeeping.
//
// Sources cited as [P1]/[P2] (page title, then the section):
//   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#pragma once
#include "device.hpp"

namespace cskv {
namespace {

constexpr int kDim = 576;          // entry dims handled by these kernels (512 latent + 64 RoPE)
constexpr int kAppendThreads = kDim;  // quantiser: one channel per thread, 9 waves
// Appends with a compressor and at least this many rows (grouped by cu_new)
// take the planned, tiled path; smaller ones the wave-per-output kernel.
constexpr int kTiledMinRows = 512;

struct AppendArgs {
    cskv_cache c;
    const float *tokens;
    const int32_t *cu_new;
    const float *w_comp;
    const uint16_t *idx_rows;
    float *ent;          // compressor output, [total_new][dim] (rows that complete an entry)
    int64_t total_new;
    // one row per sequence only: this row's window entry, written with the append
    uint16_t *swa_ring;  // [batch][swa_window][dim] bf16, or null
    const float *swa_rows;
    int swa_window;
    // one row per sequence, entry written after the head kernel: the cache
    // row of each sequence's new entry, -1 for none (written by the head)
    int64_t *slots;
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

// (b is row r's sequence and p its token count, read by the caller so that
// it can issue other loads before waiting for them.)
template <bool kCompress>
__device__ __forceinline__ RowInfo row_info(const AppendArgs &a, int64_t r, int b, int64_t p)
{
    const cskv_cache &c = a.c;
    RowInfo ri{b, -1, -1};
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    const int64_t q = r - row0;
    if (p < 0 || !rows_ok(row0, m, a.total_new) || q < 0 || q >= m) return ri;
    if (kCompress) {
        const int64_t pos = p + q;
        if ((pos & 1) == 0) return ri;                 // first half of a pair
        if ((p + m) / 2 > c.capacity) return ri;       // rejected sequence (finalize flags it)
        ri.entry = pos >> 1;
        ri.partner = q > 0 ? r - 1 : -1;
    } else {
        const int rt = c.ratio;                        // tokens per entry
        if ((p % rt) != 0 || p / rt + m > c.capacity) return ri;
        ri.entry = p / rt + q;
    }
    return ri;
}

// ---------------------------------------------------------------- compressor

// Stand-in 2->1 compressor [P2 三、"突破四" (2 tokens -> 1 entry); P1 §3.2]:
// e[ch] = sum_j W[ch][j] u[j], u = x_even || x_odd, in a fixed fp32 order:
// the 1152 terms are cut into 64 blocks of 18, each folded upward from +0
// with one fused multiply-add per term, and the 64 block sums are added as a
// pairwise tree (blocks 2i and 2i+1 first).  The tiled kernel of large appends
// cuts the tree at its level-3 nodes instead (see there).
constexpr int kCompTerms = 2 * kDim / kWave;     // 18 terms per block

// Small appends (a decode step): lane l of a wave owns block l; it keeps
// u's 18 terms of E input rows in registers and reads W[ch][18 l ..
// 18 l + 17], so the wave reads each W row contiguously once for all E
// rows.  The tree is four DPP steps inside each row of 16 lanes (lane p
// adds lane p + w) and one scalar step over the four row sums.  A wave
// takes `cpw` output channels of E consecutive input rows.  Its loads are
// issued in three groups before any is waited for: the rows' token counts,
// the W rows of up to kDepth channels (they depend on nothing), then the
// token rows (their addresses depend on the counts).
constexpr int kDppRowShl = 0x100;

template <int CTRL>
__device__ __forceinline__ float dpp_shl(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}


// One output of the compressor for one input row, held across the wave:
// lane l's 18 terms u (its block of u = x_even || x_odd) against the same
// block of the output's W row w, folded upward from +0 with one fused
// multiply-add per term, then the pairwise tree over the 64 block sums.
// The result is in every lane.
__device__ __forceinline__ float compress_dot(const float2 (&w)[kCompTerms / 2], const float (&u)[kCompTerms])
{
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < kCompTerms / 2; ++t) {
        acc = fmaf(w[t].x, u[2 * t], acc);
        acc = fmaf(w[t].y, u[2 * t + 1], acc);
    }
    acc = acc + dpp_shl<kDppRowShl | 1>(acc);
    acc = acc + dpp_shl<kDppRowShl | 2>(acc);
    acc = acc + dpp_shl<kDppRowShl | 4>(acc);
    acc = acc + dpp_shl<kDppRowShl | 8>(acc);
    const float q0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
    const float q1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 16));
    const float q2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 32));
    const float q3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 48));
    return (q0 + q1) + (q2 + q3);
}

template <int E>
__device__ __forceinline__ void compress_wave(const AppendArgs &a, int cpw, int bx, int by)
{
    constexpr int kDepth = E <= 4 ? 6 : 3;         // W rows in flight per wave
    constexpr int kH = kCompTerms / 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r0 = (int64_t)by * E;
    const int c0 = bx * cpw;
    const int c1 = c0 + cpw < kDim ? c0 + cpw : kDim;

    int bs[E];
    int64_t ps[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t r = r0 + e < a.total_new ? r0 + e : r0;
        bs[e] = seq_of_row(a.cu_new, a.c.batch, (int)r);
        ps[e] = a.c.n_tokens[bs[e]];
    }
    const float2 *wl = reinterpret_cast<const float2 *>(a.w_comp) + kH * lane;
    float2 w[kDepth][kH];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        const int c = c0 + d < c1 ? c0 + d : c1 - 1;
#pragma unroll
        for (int t = 0; t < kH; ++t) w[d][t] = wl[(size_t)c * kDim + t];
    }

    // u's terms of this lane's block for every row of the group that
    // completes an entry; lanes 0-31 hold x_even, lanes 32-63 x_odd (rows
    // that complete no entry read row 0 and are never used)
    float u[E][kCompTerms];
    uint32_t act = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t r = r0 + e;
        RowInfo ri{0, -1, -1};
        if (r < a.total_new) ri = row_info<true>(a, r, bs[e], ps[e]);
        const bool on = ri.entry >= 0;
        act |= (uint32_t)on << e;
        const float *src = !on ? a.tokens
                         : lane < kWave / 2
                               ? (ri.partner >= 0 ? a.tokens + (size_t)ri.partner * kDim
                                                  : a.c.pending + (size_t)ri.b * kDim) + kCompTerms * lane
                               : a.tokens + (size_t)r * kDim + kCompTerms * (lane - kWave / 2);
#pragma unroll
        for (int t = 0; t < kH; ++t) {
            const float2 x = reinterpret_cast<const float2 *>(src)[t];
            u[e][2 * t] = x.x;
            u[e][2 * t + 1] = x.y;
        }
    }
    if (act == 0) return;

    for (int cb = c0; cb < c1; cb += kDepth) {
        if (cb != c0) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int c = cb + d < c1 ? cb + d : c1 - 1;
#pragma unroll
                for (int t = 0; t < kH; ++t) w[d][t] = wl[(size_t)c * kDim + t];
            }
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int c = cb + d;
            if (c >= c1) break;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (!((act >> e) & 1u)) continue;
                const float res = compress_dot(w[d], u[e]);
                if (lane == e) a.ent[(size_t)(r0 + e) * kDim + c] = res;
            }
        }
    }
}

// The compressor of a decode step whose head kernel has advanced the token
// counts (one row per sequence, a.slots recorded), one wave: a row completes
// an entry exactly when its slot is recorded, its partner being the pending
// token.  The wave takes output channels [CPW bx, CPW bx + CPW) and RG groups
// of E rows in turn, rows [E (RG by + g), E (RG by + g) + E) for g < RG: the
// W rows are loaded once, then per group the slots and the rows' terms, all
// before the group's first wait.  Same arithmetic as compress_wave
// (compress_dot).
template <int E, int CPW, int RG>
__device__ __forceinline__ void compress_wave_slots(const AppendArgs &a, int bx, int by)
{
    constexpr int kH = kCompTerms / 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int c0 = bx * CPW;
    // only the sign of a slot matters: its high word (little-endian int64)
    const int32_t *slot_hi = reinterpret_cast<const int32_t *>(a.slots) + 1;
    const float2 *wl = reinterpret_cast<const float2 *>(a.w_comp) + kH * lane;
    float2 w[CPW][kH];
#pragma unroll
    for (int d = 0; d < CPW; ++d) {
        const int c = c0 + d < kDim ? c0 + d : kDim - 1;
#pragma unroll
        for (int t = 0; t < kH; ++t) w[d][t] = wl[(size_t)c * kDim + t];
    }
    for (int g = 0; g < RG; ++g) {
        const int r0 = (by * RG + g) * E;
        if (r0 >= a.total_new) break;
        int32_t sl[E];
#pragma unroll
        for (int e = 0; e < E; ++e) sl[e] = slot_hi[2 * (r0 + e < a.total_new ? r0 + e : r0)];
        float u[E][kCompTerms];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int r = r0 + e < a.total_new ? r0 + e : r0;   // a row past the batch reads row r0, unused
            const float *src = lane < kWave / 2 ? a.c.pending + (size_t)r * kDim + kCompTerms * lane
                                                : a.tokens + (size_t)r * kDim + kCompTerms * (lane - kWave / 2);
#pragma unroll
            for (int t = 0; t < kH; ++t) {
                const float2 x = reinterpret_cast<const float2 *>(src)[t];
                u[e][2 * t] = x.x;
                u[e][2 * t + 1] = x.y;
            }
        }
        uint32_t act = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) act |= (uint32_t)(r0 + e < a.total_new && sl[e] >= 0) << e;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (!((act >> e) & 1u)) continue;
#pragma unroll
            for (int d = 0; d < CPW; ++d) {
                const float res = compress_dot(w[d], u[e]);
                if (lane == 0 && c0 + d < kDim) a.ent[(size_t)(r0 + e) * kDim + c0 + d] = res;
            }
        }
    }
}

template <int E>
__global__ __launch_bounds__(kWave) void compress_kernel(AppendArgs a, int cpw)
{
    compress_wave<E>(a, cpw, blockIdx.x, blockIdx.y);
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

// fp32 -> OCP E4M3 byte [P2 四、"P4 main KV" (window rows kept in FP8)]: the
// nearest E4M3 value, ties to the even mantissa, magnitudes past 448
// saturating to 448, sign kept.  Normal results round the fp32 mantissa to 3
// bits; below 2^-6 the value is a multiple of 2^-9, rounded with rintf.
__device__ __forceinline__ uint32_t e4m3_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a < 448.0f)) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);     // 0..8 (8 = 2^-6, code 0x08)
    const uint32_t au = __float_as_uint(a);
    uint32_t e = (au >> 23) - 127 + 7, m = (au >> 20) & 7u;
    const uint32_t rem = au & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) {
        if (++m == 8u) { m = 0; ++e; }
    }
    const uint32_t code = (e << 3) | m;
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Indexer key in the pages' FP4 form [P2 四、"890 字节是怎么算出来的" (72 B per
// 128-dim key); P2 四、"P4 main KV" (E2M1, one 8-bit scale per 16 channels)]:
// thread t < Di holds dim t of the bf16 row.  Each 16-dim group takes the
// E8M0 scale 2^(floor(log2 amax) - 2) (byte 0 and zero codes when amax = 0);
// codes are the nearest E2M1 of x / scale (exact: a power of two).  Called by
// whole waves (Di is a multiple of 64).
__device__ void quantize_idx_fp4(float x, int t, uint8_t *codes_row, uint8_t *scales_row)
{
    float a = fabsf(x);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
    int e = -127;
    if (a > 0.0f) {
        int ex;
        (void)frexpf(a, &ex);                      // a = m 2^ex, 0.5 <= m < 1
        e = ex - 1 - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    uint32_t code = a > 0.0f ? e2m1_code(ldexpf(x, -e)) : 0u;
    code |= __shfl_down(code, 1) << 4;             // 2 codes (even t)
    code |= __shfl_down(code, 2) << 8;             // 4 codes
    code |= __shfl_down(code, 4) << 16;            // 8 codes
    if ((t & 7) == 0) *reinterpret_cast<uint32_t *>(codes_row + (t >> 1)) = code;
    if ((t & 15) == 0) scales_row[t >> 4] = (uint8_t)(e + 127);
}

// The pages' main-entry form [P2 四、"P4 main KV" (E2M1, one 8-bit scale per
// 16 channels)]: channel t of a row of n; each 16-channel group (inside one
// wave) takes the E8M0 scale 2^(floor(log2 amax) - 2), byte 0 and zero codes
// when amax = 0.  Called by all threads of the block.
__device__ void quantize_channel_mx16(float x, int t, int n, uint8_t *codes_row, uint8_t *scales_row)
{
    const bool live = t < n;
    float a = live ? fabsf(x) : 0.0f;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
    int e = -127;
    if (a > 0.0f) {
        int ex;
        (void)frexpf(a, &ex);
        e = ex - 1 - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    uint32_t code = (live && a > 0.0f) ? e2m1_code(ldexpf(x, -e)) : 0u;
    code |= __shfl_down(code, 1) << 4;
    code |= __shfl_down(code, 2) << 8;
    code |= __shfl_down(code, 4) << 16;
    if (live && (t & 7) == 0) *reinterpret_cast<uint32_t *>(codes_row + (t >> 1)) = code;
    if (live && (t & 15) == 0) scales_row[t >> 4] = (uint8_t)(e + 127);
}

// Sequence b after its rows are quantised: store the trailing odd token,
// advance n_tokens, or flag a rejected sequence.  p is n_tokens[b] as the
// append found it.  Returns the sequence's token count afterwards.
template <bool kCompress>
__device__ int64_t finalize_seq(const AppendArgs &a, int b, int64_t p, int t, int nthreads)
{
    const cskv_cache &c = a.c;
    const int64_t row0 = a.cu_new ? a.cu_new[b] : b;
    const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
    if (m == 0) return p;
    if (p < 0 || !rows_ok(row0, m, a.total_new)) {
        if (t == 0) atomicOr(c.status, CSKV_STATUS_BAD_STATE);
        return p;
    }
    if (kCompress) {
        if ((p + m) / 2 > c.capacity) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_OVERFLOW);
            return p;
        }
        if (((p + m) & 1) != 0) {
            const float *last = a.tokens + (size_t)(row0 + m - 1) * kDim;
            for (int i = t; i < kDim; i += nthreads) c.pending[(size_t)b * kDim + i] = last[i];
        }
        if (t == 0) c.n_tokens[b] = (int32_t)(p + m);
        return p + m;
    } else {
        const int rt = c.ratio;
        if ((p % rt) != 0) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_ODD_ENTRY_APPEND);
            return p;
        }
        if (p / rt + m > c.capacity) {
            if (t == 0) atomicOr(c.status, CSKV_STATUS_OVERFLOW);
            return p;
        }
        if (t == 0) c.n_tokens[b] = (int32_t)(p + rt * m);
        return p + rt * m;
    }
}

// Quantise entry value e (channel t of the entry) into cache slot `slot`
// (sequence-major row of every plane) and copy or quantise the indexer key
// there (key_t: dim t of the key row, for t < idx_dim).  Called by all threads of a kAppendThreads block
// (barriers inside).
__device__ __forceinline__ void quantize_main(const AppendArgs &a, float e, int t, size_t slot, float *wave_max)
{
    const cskv_cache &c = a.c;
    if (c.k_format == CSKV_KV_MX16) {
        quantize_channel_mx16(e, t, kDim, c.k_codes + slot * (kDim / 2),
                              reinterpret_cast<uint8_t *>(c.k_scales) + slot * (kDim / 16));
        if (c.v_group > 0) {
            const int dv = c.dim - c.rope_dim;
            quantize_channel_mx16(e, t, dv, c.v_codes + slot * (dv / 2),
                                  reinterpret_cast<uint8_t *>(c.v_scales) + slot * (dv / 16));
        }
    } else {
        quantize_channel(e, t, kDim, c.k_group, c.k_codes + slot * (kDim / 2),
                         c.k_scales + slot * (kDim / c.k_group), wave_max);
        if (c.v_group > 0) {
            const int dv = c.dim - c.rope_dim;
            quantize_channel(e, t, dv, c.v_group, c.v_codes + slot * (dv / 2),
                             c.v_scales + slot * (dv / c.v_group), wave_max);
        }
    }
}

__device__ __forceinline__ void store_idx_key(const AppendArgs &a, int t, size_t slot, uint16_t key_t)
{
    const cskv_cache &c = a.c;
    if (c.idx_format == CSKV_IDX_FP4) {
        if (t < c.idx_dim)                      // whole waves: idx_dim is 64 or 128
            quantize_idx_fp4(bf16_bits_to_f32(key_t), t,
                             reinterpret_cast<uint8_t *>(c.idx_keys) + slot * (c.idx_dim / 2),
                             c.idx_scales + slot * (c.idx_dim / 16));
    } else if (t < c.idx_dim) {
        c.idx_keys[slot * c.idx_dim + t] = key_t;
    }
}

__device__ __forceinline__ void quantize_entry(const AppendArgs &a, float e, int t, size_t slot, uint16_t key_t,
                                               float *wave_max)
{
    quantize_main(a, e, t, slot, wave_max);
    store_idx_key(a, t, slot, key_t);
}

// quantize_main for a block of 512 threads: thread t holds channel t (every
// value channel and the first 512 key channels, wave_max for 8 waves), wave 0
// also channel 512 + t of the key plane (groups of at most 64 channels lie
// inside one wave).  e_row: the entry's kDim channels.
__device__ __forceinline__ void quantize_main_512(const AppendArgs &a, const float *e_row, int t, size_t slot,
                                                  float *wave_max)
{
    static_assert(kDim - 512 <= kWave, "one wave takes the channels past 512");
    const cskv_cache &c = a.c;
    const float x0 = e_row[t], x1 = e_row[512 + (t & (kWave - 1))];
    if (c.k_format == CSKV_KV_MX16) {
        uint8_t *kc = c.k_codes + slot * (kDim / 2), *ks = reinterpret_cast<uint8_t *>(c.k_scales) + slot * (kDim / 16);
        quantize_channel_mx16(x0, t, kDim, kc, ks);
        if (t < kWave) quantize_channel_mx16(x1, 512 + t, kDim, kc, ks);
        if (c.v_group > 0) {
            const int dv = c.dim - c.rope_dim;
            quantize_channel_mx16(x0, t, dv, c.v_codes + slot * (dv / 2),
                                  reinterpret_cast<uint8_t *>(c.v_scales) + slot * (dv / 16));
        }
    } else {
        uint8_t *kc = c.k_codes + slot * (kDim / 2);
        float *ks = c.k_scales + slot * (kDim / c.k_group);
        quantize_channel(x0, t, kDim, c.k_group, kc, ks, wave_max);
        if (t < kWave) quantize_channel(x1, 512 + t, kDim, c.k_group, kc, ks, wave_max);
        if (c.v_group > 0) {
            const int dv = c.dim - c.rope_dim;
            quantize_channel(x0, t, dv, c.v_group, c.v_codes + slot * (dv / 2),
                             c.v_scales + slot * (dv / c.v_group), wave_max);
        }
    }
}

}  // namespace
}  // namespace cskv
