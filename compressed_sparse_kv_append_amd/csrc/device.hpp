// device.hpp -- gfx950 device helpers shared by the kernels of this library.
//
// Sources cited as [P1]/[P2] (page title, then the section):
//   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#pragma once
#include <hip/hip_runtime.h>

#include "cskv.h"
#include <stdint.h>

namespace cskv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

// fp32 -> bf16 bits, round to nearest, ties to even mantissa (finite input).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---------------------------------------------------------------- E2M1

// E2M1 code of v [P1 §3.1; P2 四、"P4 main KV"]: the magnitude code counts the
// rounding thresholds v passes.  Midpoints that round down to an even code use
// '>', midpoints that round up to an even code use '>='; past 5 everything
// rounds to 6 (saturation).  Sign bit 3 follows the sign of v.
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    float m = fabsf(v);
    uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                 (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
                 (uint32_t)(m > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// bf16 bit pattern of an E2M1 code's value (exact: every E2M1 value has at
// most 2 significant bits).  Magnitudes 0, .5, 1, 1.5 | 2, 3, 4, 6.
__device__ __forceinline__ uint32_t e2m1_to_bf16_bits(uint32_t code)
{
    const uint64_t lo = 0x3FC03F803F000000ull;   // codes 0..3
    const uint64_t hi = 0x40C0408040404000ull;   // codes 4..7
    uint32_t m = code & 7u;
    uint64_t t = (m & 4u) ? hi : lo;
    uint32_t mag = (uint32_t)(t >> (16u * (m & 3u))) & 0xFFFFu;
    return mag | ((code & 8u) << 12);
}

// Eight codes (one 32-bit word, low nibble first) -> eight bf16 values packed
// two per 32-bit word in channel order.
__device__ __forceinline__ u32x4_t e2m1x8_to_bf16x8(uint32_t w)
{
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t a = e2m1_to_bf16_bits((w >> (8 * i)) & 0xFu);
        uint32_t b = e2m1_to_bf16_bits((w >> (8 * i + 4)) & 0xFu);
        r[i] = a | (b << 16);
    }
    return r;
}

// ---------------------------------------------------------------- MFMA

// D = A * B + C for 16x16 tiles with a 32-deep bf16 contraction.
// Operand layout (lane l): A row l%16, B column l%16, contraction slots
// 8*(l/16) .. 8*(l/16)+7; result D[4*(l/16)+v][l%16] in element v.
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t &a, const u32x4_t &b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave scans

// Cross-lane steps through DPP (no LDS round trip): row_shr:n moves values n
// lanes up inside each row of 16; row_bcast:15 / row_bcast:31 carry lane 15
// (31) of a row into the next row(s).  Lanes without a source take `ident`.
enum : int { kDppRowShr = 0x110, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143 };

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t ident, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix (op = add, max or min) over the 64 lanes of the wave.
template <class Op>
__device__ __forceinline__ uint32_t wave_inclusive(uint32_t v, uint32_t ident, Op op)
{
    v = op(v, dpp_u32<kDppRowShr | 1, 0xF>(ident, v));
    v = op(v, dpp_u32<kDppRowShr | 2, 0xF>(ident, v));
    v = op(v, dpp_u32<kDppRowShr | 4, 0xF>(ident, v));
    v = op(v, dpp_u32<kDppRowShr | 8, 0xF>(ident, v));
    v = op(v, dpp_u32<kDppRowBcast15, 0xA>(ident, v));
    v = op(v, dpp_u32<kDppRowBcast31, 0xC>(ident, v));
    return v;
}

__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v)
{
    return wave_inclusive(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Reductions over the wave, the same value in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = wave_inclusive(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = wave_inclusive(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v)
{
    v = wave_inclusive(v, 0u, [](uint32_t a, uint32_t b) { return a | b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v)
{
    v = wave_inclusive(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a & b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// ---------------------------------------------------------------- misc

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key).
// -0 is folded into +0 first so equal scores give equal keys.
// E8M0 byte -> the fp32 power of two it encodes (byte 0: 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b)
{
    return __uint_as_float(b ? b << 23 : 0x00400000u);
}

// Eight E2M1 codes (one word, low nibble first) times a power of two ->
// eight bf16 values; exact, E2M1 values having at most two significant bits.
__device__ __forceinline__ u32x4_t fp4x8_scaled_to_bf16x8(uint32_t w, float scale)
{
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return r;
}

__device__ __forceinline__ uint32_t score_key(float s)
{
    s = s + 0.0f;
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Plane row of entry e of sequence b: [batch][capacity] planes, or paged
// planes [n_pages][page_size] through the sequence's block table (-1 for a
// table entry outside [0, n_pages)).
__device__ __forceinline__ int64_t plane_row(const cskv_cache &c, int b, int64_t e)
{
    if (c.page_size <= 0) return (int64_t)b * c.capacity + e;
    const int sh = __builtin_ctz(c.page_size);
    const int32_t pg = c.block_table[(size_t)b * c.max_pages + (e >> sh)];
    return pg >= 0 && pg < c.n_pages ? ((int64_t)pg << sh) + (e & (c.page_size - 1)) : -1;
}

// Raw buffer resources: a load or store whose offset (plus its size) passes
// num_records does not touch memory (a load returns zeros), so a lane can be
// masked by its offset alone and every lane executes the same instructions.
constexpr uint32_t kMasked = 0x80000000u;    // offset past the end of every resource
constexpr int kRsrcWord3 = 0x00020000;       // raw 32-bit buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ int64_t entries_of(const int32_t *n_tokens, int b, int capacity, int ratio)
{
    int64_t e = (int64_t)n_tokens[b] / ratio;
    e = e < 0 ? 0 : e;
    return e > capacity ? capacity : e;
}

// Sequence owning input row r: cu_new == nullptr means row r is sequence r.
__device__ __forceinline__ int seq_of_row(const int32_t *cu_new, int batch, int r)
{
    if (!cu_new) return r;
    int lo = 0, hi = batch - 1;      // last b with cu_new[b] <= r
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_new[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace cskv
