// attention.hip -- gather + dequantise + one softmax over the selected
// compressed entries and the window rows, for all query heads of a sequence
// [P2 三、"突破四：滑动窗口和稀疏注意力" (sparse global branch + 128-token
// window); P2 三、"突破二：MLA，低秩压缩" (every head reads the same latent
// entry); P2 四、"P4 main KV" (FP4 is storage only; dequantise before use)].
//
// Work decomposition.  The keys of a sequence are the k selected entries,
// cut into chunks of 128, and the window rows, cut into chunks of 64.  A
// split is a run of entry chunks and/or a run of window chunks; one block of
// 8 waves takes 16 query heads and one split, and a second kernel merges the
// partial softmaxes of each head by their log-sum-exp (skipped when there is
// one split).  A split may mix the kinds so that every block of a launch
// carries about the same work.  The blocks that share a split's keys (one
// per head group) are numbered so that they land on the same XCD and read
// the gathered rows through one L2.  Each kind has a loop of its own, run one
// after the other with one softmax state, so that each loop holds its own
// prefetch registers and every load in it is unconditional.
//
// Per chunk.  The gathered rows stay E2M1 codes in LDS: the key plane row-
// major (MFMA B operand of Q.K^T: 8 consecutive dims of one key = one 32-bit
// word of codes) and the value plane transposed to [dim][key] nibbles (B
// operand of P.V: 8 consecutive keys of one dim = one word), the transpose
// done in registers on the way from HBM to LDS.  Each operand word becomes 8
// bf16 values with four hardware FP4 conversions; E2M1 values are exact in
// bf16.  Group scales stay fp32 outside the MFMA: per key group on the
// logits, folded into the probabilities per value group.  q and the scaled
// probabilities are each split into bf16 high and low parts, so the products
// carry about 16 significant bits.  Window rows are bf16 already and are
// staged row-major.  The softmax runs online in base 2 with fp32 statistics.
// The next chunk's HBM reads are issued before the current chunk is computed.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace cskv {

namespace {

constexpr int kThreads = 512;                 // 8 waves
constexpr int kHG = 16;                       // query heads per block (one MFMA row tile)
constexpr int kSK = 128;                      // selected entries per chunk
constexpr int kWK = 64;                       // window rows per chunk
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kSteps = kD / 32;               // 18 contraction steps of Q.K^T
constexpr int kHalf = kSteps / 2;
constexpr int kMaxKG = kD / 32;
constexpr int kMaxVG = kDv / 32;
// Key-code row stride in words: 72 + 2, so the 16 rows of a key tile start on
// 16 distinct even banks and one 32-bit operand read per lane is conflict-free.
constexpr int kKcRow = kD / 8 + 2;
// Transposed value codes: per 32-key group, dim d's 4 words (8 keys each) sit
// at (d / 8) * 33 + 4 * (d % 8); the odd octet stride spreads the transpose
// writes of 32 lanes (one dim octet each) over 32 banks.
constexpr int kVtOct = 33;
constexpr int kVtGroup = (kDv / 8) * kVtOct;
constexpr int kWinRow = kD + 8;               // 584 bf16 per staged window row
constexpr int kSRow = kSK + 4;                // floats per head row of logits / probabilities
constexpr int kMaxSplitChunks = 8;            // chunks a block keeps key sources for

struct SparseStage {
    uint32_t kc[kSK * kKcRow];                // key-plane codes, row-major
    uint32_t vt[(kSK / 32) * kVtGroup];       // value codes, [32-key group][dim][8-key word]
};
struct WindowStage {
    uint16_t kr[kWK][kWinRow];                // window rows, bf16
};

struct AttnSmem {
    union {
        SparseStage sp;
        WindowStage win;
    } st;
    u32x4_t q[kSteps][2][kWave];              // q hi / lo: MFMA A operand per step and lane
    float ks[kMaxKG][kSK];                    // key-plane scale per group and key
    float vs[kMaxVG][kSK];                    // value-plane scale per group and key (split planes)
    float s[2][kHG][kSRow];                   // logits (two contraction halves), then probabilities
    float m[kHG], l[kHG], alpha[kHG];
    int32_t src[kMaxSplitChunks * kSK];       // entry index / window slot per key, -1 masked
};

struct AttnArgs {
    cskv_cache c;
    const float *q;
    const int32_t *idx;
    const uint16_t *swa;
    const int32_t *swa_len;
    float *out;
    float *lse;
    float *part_o;      // [B][HG][S][16][512] unnormalised partial outputs (S > 1)
    float *part_ml;     // [B][HG][S][2][16] partial max (log2 units) and sum
    int heads, k, window;
    int n_sparse, n_win;
    int win_split0, per_sparse, per_win, splits;
    float scale_log2;   // softmax_scale * log2(e)
};

// Per-block constants shared by the chunk loop.
struct Ctx {
    int t, lane, w, col, grp;
    int ne, nw;         // entry chunks, then window chunks, of this block
    int G;              // key groups per row
    size_t row0;        // first plane row of the sequence's buffer resources (0 for paged planes)
    uint32_t rows;      // plane rows those resources cover (the capacity, or every paged row)
    const uint8_t *ring;    // this sequence's window rows (bf16, or FP8 E4M3 bytes)
};

__device__ __forceinline__ u32x4_t lds16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// Eight E2M1 codes (one word, low nibble first) -> eight bf16 values.
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t w)
{
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even), packed low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// hi/lo bf16 split of 8 floats: x = hi + lo + O(2^-17 |x|)
__device__ __forceinline__ void split8(const float *x, u32x4_t &hi, u32x4_t &lo)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        hi[i] = h;
        lo[i] = pack_bf16x2(x[2 * i] - __uint_as_float(h << 16), x[2 * i + 1] - __uint_as_float(h & 0xFFFF0000u));
    }
}

// 8x8 transpose of 4-bit codes: in[j] holds dims 0..7 of key j (nibble d);
// out[d] holds keys 0..7 of dim d (nibble j).  Three stages swap the
// off-diagonal 4x4, 2x2 and 1x1 blocks.
__device__ __forceinline__ void transpose_nibbles(const uint32_t (&in)[8], uint32_t (&out)[8])
{
    uint32_t a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = in[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t x = a[j], y = a[j + 4];
        a[j] = (x & 0x0000FFFFu) | (y << 16);
        a[j + 4] = (x >> 16) | (y & 0xFFFF0000u);
    }
#pragma unroll
    for (int j = 0; j < 8; j += 4)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t x = a[j + i], y = a[j + i + 2];
            a[j + i] = (x & 0x00FF00FFu) | ((y & 0x00FF00FFu) << 8);
            a[j + i + 2] = ((x >> 8) & 0x00FF00FFu) | (y & 0xFF00FF00u);
        }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const uint32_t x = a[j], y = a[j + 1];
        a[j] = (x & 0x0F0F0F0Fu) | ((y & 0x0F0F0F0Fu) << 4);
        a[j + 1] = ((x >> 4) & 0x0F0F0F0Fu) | (y & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) out[d] = a[d];
}

// One chunk's HBM reads, held in registers until they are written to LDS.
// They are buffer loads against a per-sequence resource: offsets are 32-bit,
// and a masked key is given an offset past the end of the resource, which the
// hardware answers with zeros, so no load waits behind a branch and masked
// keys arrive with zero codes and zero scales.
struct SparseRegs {
    uint32_t v[16];     // value-plane words of key octets w and w + 8, word = lane
    u32x4_t k[5];       // split planes: 16-byte pieces of key codes; one plane: k[0].xy = rope words
    float sc[9];        // key scales 0-4, value scales 5-8 (group t / 128 + 4 i, key t % 128)
};
struct WindowRegs {
    u32x4_t p[9];       // 64 rows x 72 pieces of 16 bytes
};

__device__ __forceinline__ uint32_t row_off(int32_t e, uint32_t row_bytes)
{
    return e >= 0 ? (uint32_t)e * row_bytes : kMasked;
}

// KG = 16: the pages' scale form (CSKV_KV_MX16): one E8M0 byte per 16
// channels, key rows of 36 bytes and value rows of 32; the scale words are
// loaded raw and spread to bytes in LDS ([group][key], in the ks / vs space).
template <bool SPLIT, int VGS, int KG>
__device__ __forceinline__ void fetch_sparse(const AttnArgs &a, const AttnSmem &sm, const Ctx &x, int lc,
                                             SparseRegs &r)
{
    const cskv_cache &c = a.c;
    const int32_t *src = sm.src + lc * kSK;
    constexpr int VG = kDv / VGS;
    constexpr uint32_t kVRowBytes = SPLIT ? kDv / 2 : kD / 2;
    const uint32_t cap = x.rows;
    const __amdgpu_buffer_rsrc_t vr =
        make_rsrc((SPLIT ? c.v_codes : c.k_codes) + x.row0 * kVRowBytes, cap * kVRowBytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(c.k_codes + x.row0 * (kD / 2), cap * (kD / 2));
    const __amdgpu_buffer_rsrc_t ksr = make_rsrc(c.k_scales + x.row0 * x.G, cap * x.G * 4);
    int32_t e[16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int4 s0 = *reinterpret_cast<const int4 *>(src + 8 * (x.w + 8 * i));
        const int4 s1 = *reinterpret_cast<const int4 *>(src + 8 * (x.w + 8 * i) + 4);
        e[8 * i + 0] = s0.x; e[8 * i + 1] = s0.y; e[8 * i + 2] = s0.z; e[8 * i + 3] = s0.w;
        e[8 * i + 4] = s1.x; e[8 * i + 5] = s1.y; e[8 * i + 6] = s1.z; e[8 * i + 7] = s1.w;
    }
    const int32_t es = src[x.t & (kSK - 1)];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        r.v[j] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(row_off(e[j], kVRowBytes) + 4 * x.lane), 0, 0);
    if (!SPLIT) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {                      // rope words 64..71 of 128 rows
            const int task = x.t + kThreads * i;
            const uint32_t off = row_off(src[task >> 3], kD / 2) + 4 * (64 + (task & 7));
            r.k[0][i] = __builtin_amdgcn_raw_buffer_load_b32(kr, (int)off, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 5; ++i) {                      // 128 rows x 18 pieces of key codes
            const int task = min(x.t + kThreads * i, kSK * 18 - 1), row = task / 18, p = task % 18;
            const uint32_t off = row_off(src[row], kD / 2) + 16 * p;
            r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off, 0, 0);
        }
    }
    if constexpr (KG == 16) {
        constexpr uint32_t kKRow = kD / 16, kVRow = kDv / 16;          // scale bytes per row
        const __amdgpu_buffer_rsrc_t kb8 =
            make_rsrc(reinterpret_cast<const uint8_t *>(c.k_scales) + x.row0 * kKRow, cap * kKRow);
        const uint32_t so = row_off(es, kKRow);
#pragma unroll
        for (int i = 0; i < 3; ++i) {                      // dwords t / 128 + 4 i of 9
            const int d = min((x.t >> 7) + 4 * i, (int)kKRow / 4 - 1);
            r.sc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kb8, (int)(so + 4 * d), 0, 0));
        }
        if (SPLIT) {
            const __amdgpu_buffer_rsrc_t vb8 =
                make_rsrc(reinterpret_cast<const uint8_t *>(c.v_scales) + x.row0 * kVRow, cap * kVRow);
            const uint32_t vo = row_off(es, kVRow);
#pragma unroll
            for (int i = 0; i < 2; ++i) {                  // dwords t / 128 + 4 i of 8
                const int d = (x.t >> 7) + 4 * i;
                r.sc[5 + i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vb8, (int)(vo + 4 * d), 0, 0));
            }
        }
        return;
    }
    const uint32_t so = row_off(es, 4 * x.G);
#pragma unroll
    for (int i = 0; i < 5; ++i) {                          // key scales: group t / 128 + 4 i
        const int g = min((x.t >> 7) + 4 * i, x.G - 1);
        r.sc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksr, (int)(so + 4 * g), 0, 0));
    }
    if (SPLIT) {
        const __amdgpu_buffer_rsrc_t vsr = make_rsrc(c.v_scales + x.row0 * VG, cap * VG * 4);
        const uint32_t vo = row_off(es, 4 * VG);
#pragma unroll
        for (int i = 0; i < 4; ++i) {                      // value scales: group t / 128 + 4 i < 16
            const int g = min((x.t >> 7) + 4 * i, VG - 1);
            r.sc[5 + i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vsr, (int)(vo + 4 * g), 0, 0));
        }
    }
}

template <bool SPLIT, int VGS, int KG>
__device__ __forceinline__ void store_sparse(AttnSmem &sm, const Ctx &x, const SparseRegs &r)
{
    constexpr int VG = kDv / VGS;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int o = x.w + 8 * i;
        uint32_t in[8], tw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) in[j] = r.v[8 * i + j];
        if (!SPLIT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sm.st.sp.kc[(8 * o + j) * kKcRow + x.lane] = in[j];
        }
        transpose_nibbles(in, tw);
        uint32_t *vt = sm.st.sp.vt + (o >> 2) * kVtGroup + x.lane * kVtOct + (o & 3);
#pragma unroll
        for (int d = 0; d < 8; ++d) vt[4 * d] = tw[d];
    }
    if (!SPLIT) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int task = x.t + kThreads * i;
            sm.st.sp.kc[(task >> 3) * kKcRow + 64 + (task & 7)] = r.k[0][i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int task = x.t + kThreads * i, row = task / 18, p = task % 18;
            if (task < kSK * 18) {
                uint2 *dst = reinterpret_cast<uint2 *>(sm.st.sp.kc + row * kKcRow + 4 * p);
                dst[0] = make_uint2(r.k[i][0], r.k[i][1]);
                dst[1] = make_uint2(r.k[i][2], r.k[i][3]);
            }
        }
    }
    const int key = x.t & (kSK - 1);
    if constexpr (KG == 16) {
        uint8_t *kb = reinterpret_cast<uint8_t *>(&sm.ks[0][0]);            // [36][kSK] bytes
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int d = (x.t >> 7) + 4 * i;
            const uint32_t w = __float_as_uint(r.sc[i]);
            if (d < kD / 64) {
#pragma unroll
                for (int by = 0; by < 4; ++by) kb[(4 * d + by) * kSK + key] = (uint8_t)(w >> (8 * by));
            }
        }
        if (SPLIT) {
            uint8_t *vb = reinterpret_cast<uint8_t *>(&sm.vs[0][0]);        // [32][kSK] bytes
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int d = (x.t >> 7) + 4 * i;
                const uint32_t w = __float_as_uint(r.sc[5 + i]);
#pragma unroll
                for (int by = 0; by < 4; ++by) vb[(4 * d + by) * kSK + key] = (uint8_t)(w >> (8 * by));
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int g = (x.t >> 7) + 4 * i;
        if (g < x.G) sm.ks[g][key] = r.sc[i];
    }
    if (SPLIT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = (x.t >> 7) + 4 * i;
            if (g < VG) sm.vs[g][key] = r.sc[5 + i];
        }
    }
}

// Window rows: task (row, p) is dims 8p .. 8p+7 of a row, 16 bytes in bf16
// or 8 bytes in FP8 (W8); FP8 rows are widened to bf16 on the way to LDS
// (exact: E4M3 values have 4 significant bits), so the staged rows are bf16
// either way.
template <bool W8>
__device__ __forceinline__ void fetch_window(const AttnArgs &a, const AttnSmem &sm, const Ctx &x, int lc,
                                             WindowRegs &r)
{
    constexpr uint32_t kRowBytes = W8 ? kD : kD * 2;
    const int32_t *src = sm.src + lc * kSK;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(x.ring, (uint32_t)a.window * kRowBytes);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const int task = x.t + kThreads * i, row = task / 72, p = task % 72;
        const uint32_t off = row_off(src[row], kRowBytes) + (W8 ? 8 : 16) * p;
        if (W8) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)off, 0, 0);
            r.p[i][0] = v[0];
            r.p[i][1] = v[1];
        } else {
            r.p[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, 0);
        }
    }
}

template <bool W8>
__device__ __forceinline__ void store_window(AttnSmem &sm, const Ctx &x, const WindowRegs &r)
{
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const int task = x.t + kThreads * i, row = task / 72, p = task % 72;
        u32x4_t v = r.p[i];
        if (W8) {
            v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.p[i][0], 1.0f, false));
            v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.p[i][0], 1.0f, true));
            v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.p[i][1], 1.0f, false));
            v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.p[i][1], 1.0f, true));
        }
        *reinterpret_cast<u32x4_t *>(&sm.st.win.kr[row][8 * p]) = v;
    }
}

// Logits of one chunk.  Wave w takes contraction half w / 4 (9 steps) of two
// key tiles (selected entries: tiles 2 (w % 4) and 2 (w % 4) + 1 of 8) or of
// one (window rows: tile w % 4 of 4); the halves are added in the softmax.
// Selected entries: the MFMA accumulates the steps of one key group, whose
// scale is then applied once in fp32.
template <int KG, int HALF>
__device__ __forceinline__ void sparse_logits_half(AttnSmem &sm, const Ctx &x)
{
    constexpr int kPer = KG / 32;                  // contraction steps per key group
    const int j0 = 32 * (x.w & 3) + x.col, j1 = j0 + 16;
    const uint32_t *k0 = sm.st.sp.kc + j0 * kKcRow + x.grp;
    const uint32_t *k1 = sm.st.sp.kc + j1 * kKcRow + x.grp;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KG == 16) {
        // E8M0 scales per 16 channels: a code word (8 dims) lies inside one
        // group, so the power-of-two scale goes into the conversion (exact)
        // and the logits need no per-group scaling
        const uint8_t *kb = reinterpret_cast<const uint8_t *>(&sm.ks[0][0]);
#pragma unroll
        for (int s = 0; s < kHalf; ++s) {
            const int step = kHalf * HALF + s, g = 2 * step + (x.grp >> 1);
            const u32x4_t qh = sm.q[step][0][x.lane], ql = sm.q[step][1][x.lane];
            const u32x4_t kb0 = fp4x8_scaled_to_bf16x8(k0[4 * step], e8m0_to_f32(kb[g * kSK + j0]));
            const u32x4_t kb1 = fp4x8_scaled_to_bf16x8(k1[4 * step], e8m0_to_f32(kb[g * kSK + j1]));
            acc0 = mfma16x16x32(qh, kb0, acc0);
            acc1 = mfma16x16x32(qh, kb1, acc1);
            acc0 = mfma16x16x32(ql, kb0, acc0);
            acc1 = mfma16x16x32(ql, kb1, acc1);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sm.s[HALF][4 * x.grp + v][j0] = acc0[v];
            sm.s[HALF][4 * x.grp + v][j1] = acc1[v];
        }
        return;
    }
#pragma unroll
    for (int s = 0; s < kHalf; ++s) {
        const int step = kHalf * HALF + s;
        const u32x4_t qh = sm.q[step][0][x.lane], ql = sm.q[step][1][x.lane];
        const u32x4_t kb0 = fp4x8_to_bf16x8(k0[4 * step]);
        const u32x4_t kb1 = fp4x8_to_bf16x8(k1[4 * step]);
        p0 = mfma16x16x32(qh, kb0, p0);
        p1 = mfma16x16x32(qh, kb1, p1);
        p0 = mfma16x16x32(ql, kb0, p0);
        p1 = mfma16x16x32(ql, kb1, p1);
        if ((step + 1) % kPer == 0 || s == kHalf - 1) {       // last step of a group in this half
            const float sc0 = sm.ks[step / kPer][j0], sc1 = sm.ks[step / kPer][j1];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc0[v] = fmaf(sc0, p0[v], acc0[v]);
                acc1[v] = fmaf(sc1, p1[v], acc1[v]);
            }
            p0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            p1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        sm.s[HALF][4 * x.grp + v][j0] = acc0[v];
        sm.s[HALF][4 * x.grp + v][j1] = acc1[v];
    }
}

template <bool SPARSE, int KG>
__device__ __forceinline__ void chunk_logits(AttnSmem &sm, const Ctx &x)
{
    const int half = x.w >> 2;
    if (SPARSE) {
        if (half == 0) sparse_logits_half<KG, 0>(sm, x);
        else sparse_logits_half<KG, 1>(sm, x);
    } else {
        const int j = 16 * (x.w & 3) + x.col;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kHalf; ++s) {
            const int step = kHalf * half + s;
            const u32x4_t kb = lds16(&sm.st.win.kr[j][32 * step + 8 * x.grp]);
            acc = mfma16x16x32(sm.q[step][0][x.lane], kb, acc);
            acc = mfma16x16x32(sm.q[step][1][x.lane], kb, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.s[half][4 * x.grp + v][j] = acc[v];
    }
}

// Reductions over the 32 lanes of a half wave, the result in every lane:
// rotations inside each row of 16 (DPP), then the two rows of the half
// exchange through a swizzle.
enum : int { kDppRowRor = 0x120, kSwizzleXor16 = 0x401F };

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float half_wave_max(float v)
{
    v = fmaxf(v, dpp_f32<kDppRowRor | 8>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor | 4>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor | 2>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor | 1>(v));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16)));
}

__device__ __forceinline__ float half_wave_sum(float v)
{
    v += dpp_f32<kDppRowRor | 8>(v);
    v += dpp_f32<kDppRowRor | 4>(v);
    v += dpp_f32<kDppRowRor | 2>(v);
    v += dpp_f32<kDppRowRor | 1>(v);
    return v + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}

// Online softmax in base 2: thread t -> head t / 32, keys t % 32 + 32 i.
// Probabilities overwrite the first logit half; m, l and the rescale factor
// alpha of each head are updated by its first thread.
template <bool SPARSE>
__device__ __forceinline__ void chunk_softmax(AttnSmem &sm, const Ctx &x, int lc, float scale_log2)
{
    constexpr int NQ = (SPARSE ? kSK : kWK) / 32;
    const int h = x.t >> 5, j0 = x.t & 31;
    const int32_t *src = sm.src + lc * kSK;
    float sv[NQ];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int j = j0 + 32 * i;
        const float v = sm.s[0][h][j] + sm.s[1][h][j];
        sv[i] = src[j] >= 0 ? v * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[i]);
    }
    mx = half_wave_max(mx);
    const float m_old = sm.m[h];
    const float m_new = fmaxf(m_old, mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const float pj = exp2f(sv[i] - m_new);
        sm.s[0][h][j0 + 32 * i] = pj;
        sum += pj;
    }
    sum = half_wave_sum(sum);
    if (j0 == 0) {
        const float al = exp2f(m_old - m_new);
        sm.alpha[h] = al;
        sm.m[h] = m_new;
        sm.l[h] = sm.l[h] * al + sum;
    }
}

// P.V: wave w owns value dims [64 w, 64 w + 64) = 4 tiles of 16.  The value
// group scales of selected entries are folded into P per group.
template <bool SPARSE, bool SPLIT, int VGS>
__device__ __forceinline__ void chunk_pv(const AttnSmem &sm, const Ctx &x, f32x4_t (&o)[4])
{
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float al = sm.alpha[4 * x.grp + v];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[nt][v] *= al;
    }
    constexpr int kGroupsHere = VGS >= 64 ? 1 : 64 / VGS;   // value groups per wave
    constexpr int kTilesPerGroup = 4 / kGroupsHere;
    constexpr int NKK = (SPARSE ? kSK : kWK) / 32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const int key0 = 32 * kk + 8 * x.grp;
        const float4 p0 = *reinterpret_cast<const float4 *>(&sm.s[0][x.col][key0]);
        const float4 p1 = *reinterpret_cast<const float4 *>(&sm.s[0][x.col][key0 + 4]);
        const float pr[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int gi = 0; gi < (SPARSE ? kGroupsHere : 1); ++gi) {
            float pv[8];
            if (SPARSE && VGS == 16) {
                // E8M0 bytes [group][key] (value plane, else the key plane's
                // first 32 groups)
                const int gv = 4 * x.w + gi;
                const uint8_t *vb = reinterpret_cast<const uint8_t *>(SPLIT ? &sm.vs[0][0] : &sm.ks[0][0]);
                const uint2 sv = *reinterpret_cast<const uint2 *>(vb + gv * kSK + key0);
#pragma unroll
                for (int i = 0; i < 8; ++i)             // p * 2^(byte - 127), exact in one ldexp
                    pv[i] = ldexpf(pr[i], (int)(((i < 4 ? sv.x : sv.y) >> (8 * (i & 3))) & 0xFFu) - 127);
            } else if (SPARSE) {
                const int gv = (64 * x.w) / VGS + gi;
                const float *vsr = SPLIT ? &sm.vs[gv][key0] : &sm.ks[gv][key0];
                const float4 v0 = *reinterpret_cast<const float4 *>(vsr);
                const float4 v1 = *reinterpret_cast<const float4 *>(vsr + 4);
                pv[0] = pr[0] * v0.x; pv[1] = pr[1] * v0.y; pv[2] = pr[2] * v0.z; pv[3] = pr[3] * v0.w;
                pv[4] = pr[4] * v1.x; pv[5] = pr[5] * v1.y; pv[6] = pr[6] * v1.z; pv[7] = pr[7] * v1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = pr[i];
            }
            u32x4_t phi, plo;
            split8(pv, phi, plo);
            constexpr int kTiles = SPARSE ? kTilesPerGroup : 4;
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                const int nt = gi * kTiles + tt;
                const int dim = 64 * x.w + 16 * nt + x.col;
                u32x4_t vb;
                if (SPARSE) {
                    vb = fp4x8_to_bf16x8(sm.st.sp.vt[kk * kVtGroup + (dim >> 3) * kVtOct + 4 * (dim & 7) + x.grp]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vb[i] = (uint32_t)sm.st.win.kr[key0 + 2 * i][dim] |
                                ((uint32_t)sm.st.win.kr[key0 + 2 * i + 1][dim] << 16);
                }
                o[nt] = mfma16x16x32(phi, vb, o[nt]);
                o[nt] = mfma16x16x32(plo, vb, o[nt]);
            }
        }
    }
}

// The chunk loop of one block: the next chunk's HBM reads are in flight
// while the current chunk is computed.
template <bool SPARSE, bool SPLIT, int VGS, int KG, bool W8>
__device__ __forceinline__ void run_chunks(const AttnArgs &a, AttnSmem &sm, const Ctx &x, int first, int end,
                                           f32x4_t (&o)[4])
{
    if (SPARSE) {
        SparseRegs r;
        fetch_sparse<SPLIT, VGS, KG>(a, sm, x, first, r);
        for (int lc = first; lc < end; ++lc) {
            __syncthreads();                               // previous chunk fully consumed
            store_sparse<SPLIT, VGS, KG>(sm, x, r);
            __syncthreads();
            if (lc + 1 < end) fetch_sparse<SPLIT, VGS, KG>(a, sm, x, lc + 1, r);
            chunk_logits<true, KG>(sm, x);
            __syncthreads();
            chunk_softmax<true>(sm, x, lc, a.scale_log2);
            __syncthreads();
            chunk_pv<true, SPLIT, VGS>(sm, x, o);
        }
    } else {
        WindowRegs r;
        fetch_window<W8>(a, sm, x, first, r);
        for (int lc = first; lc < end; ++lc) {
            __syncthreads();
            store_window<W8>(sm, x, r);
            __syncthreads();
            if (lc + 1 < end) fetch_window<W8>(a, sm, x, lc + 1, r);
            chunk_logits<false, KG>(sm, x);
            __syncthreads();
            chunk_softmax<false>(sm, x, lc, a.scale_log2);
            __syncthreads();
            chunk_pv<false, SPLIT, VGS>(sm, x, o);
        }
    }
}

// VGS: the value group size in effect (the value plane's group, else the key
// plane's): 32, 64 or 128.  SPLIT: the cache has a separate value plane.
// KG: the key plane's group, 32 or 64.
// W8: the window rows are FP8 (E4M3).
template <int VGS, bool SPLIT, int KG, bool W8>
__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(AttnArgs a)
{
    __shared__ AttnSmem sm;
    const cskv_cache &c = a.c;
    const int HG = a.heads / kHG;

    // ---- block -> (sequence, head group, split); blocks of one (sequence,
    // split) share id % 8, i.e. one XCD
    const int U = c.batch * a.splits;
    const int id = blockIdx.x, xcd = id & 7, rest = id >> 3;
    const int hg = rest % HG, u = (rest / HG) * 8 + xcd;
    if (u >= U) return;
    const int b = u / a.splits, split = u % a.splits;
    // entry chunks [e0, e1) and window chunks [w0, w1) of this split
    const int e0 = min(split * a.per_sparse, a.n_sparse), e1 = min(e0 + a.per_sparse, a.n_sparse);
    const int ws = split - a.win_split0;
    const int w0 = ws < 0 ? 0 : min(ws * a.per_win, a.n_win), w1 = ws < 0 ? 0 : min(w0 + a.per_win, a.n_win);

    Ctx x;
    x.t = threadIdx.x;
    x.lane = x.t & (kWave - 1);
    x.w = x.t / kWave;
    x.col = x.lane & 15;
    x.grp = x.lane >> 4;
    x.ne = e1 - e0;
    x.nw = w1 - w0;
    x.G = kD / KG;
    const bool paged = c.page_size > 0;
    x.row0 = paged ? 0 : (size_t)b * c.capacity;
    x.rows = paged ? (uint32_t)c.n_pages * (uint32_t)c.page_size : (uint32_t)c.capacity;
    x.ring = reinterpret_cast<const uint8_t *>(a.swa) + (size_t)b * a.window * kD * (W8 ? 1 : 2);
    const int64_t E = entries_of(c.n_tokens, b, c.capacity, c.ratio);
    int64_t nswa = a.swa_len ? (int64_t)a.swa_len[b] : (int64_t)c.n_tokens[b];
    nswa = nswa < 0 ? 0 : (nswa > a.window ? a.window : nswa);

    // ---- key sources of every chunk of the split
    for (int i = x.t; i < (x.ne + x.nw) * kSK; i += kThreads) {
        const int lc = i / kSK, j = i % kSK;
        const bool sparse = lc < x.ne;
        const int chunk = sparse ? e0 + lc : w0 + lc - x.ne;
        int32_t s = -1;
        if (sparse) {
            const int jj = chunk * kSK + j;
            const int32_t e = jj < a.k ? a.idx[(size_t)b * a.k + jj] : -1;
            s = (e >= 0 && e < E) ? e : -1;
            if (paged && s >= 0) s = (int32_t)plane_row(c, b, s);    // a plane row; -1 (bad page): skipped
        } else if (j < kWK) {
            const int64_t slot = (int64_t)chunk * kWK + j;
            s = slot < nswa ? (int32_t)slot : -1;
        }
        sm.src[i] = s;
    }
    // ---- query operands of the 16 heads, hi + lo, per contraction step
    {
        const float *qbase = a.q + ((size_t)b * a.heads + kHG * hg) * kD;
        for (int i = x.t; i < kSteps * kWave; i += kThreads) {
            const int s = i / kWave, ln = i % kWave;
            const float *qr = qbase + (size_t)(ln & 15) * kD + 32 * s + 8 * (ln >> 4);
            const float4 x0 = *reinterpret_cast<const float4 *>(qr);
            const float4 x1 = *reinterpret_cast<const float4 *>(qr + 4);
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            u32x4_t hi, lo;
            split8(xv, hi, lo);
            sm.q[s][0][ln] = hi;
            sm.q[s][1][ln] = lo;
        }
    }
    if (x.t < kHG) { sm.m[x.t] = -1e30f; sm.l[x.t] = 0.f; }
    f32x4_t o[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    if (x.ne > 0) run_chunks<true, SPLIT, VGS, KG, W8>(a, sm, x, 0, x.ne, o);
    if (x.nw > 0) run_chunks<false, SPLIT, VGS, KG, W8>(a, sm, x, x.ne, x.ne + x.nw, o);
    __syncthreads();

    // ---- results: final (one split) or partial (merged by attn_merge_kernel)
    const int t = x.t, w = x.w, col = x.col, grp = x.grp;
    const size_t head0 = (size_t)b * a.heads + kHG * hg;
    if (a.splits == 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int h = 4 * grp + v;
            const float l = sm.l[h];
            const float inv = l > 0.f ? 1.0f / l : 0.f;
            float *orow = a.out + (head0 + h) * kDv + 64 * w + col;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) orow[16 * nt] = o[nt][v] * inv;
        }
        if (a.lse && t < kHG) {
            const float l = sm.l[t];
            a.lse[head0 + t] = l > 0.f ? (sm.m[t] + log2f(l)) * 0.69314718055994531f : -INFINITY;
        }
    } else {
        const size_t pidx = ((size_t)b * HG + hg) * a.splits + split;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int h = 4 * grp + v;
            float *orow = a.part_o + (pidx * kHG + h) * kDv + 64 * w + col;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) orow[16 * nt] = o[nt][v];
        }
        if (t < kHG) {
            a.part_ml[pidx * 2 * kHG + t] = sm.l[t] > 0.f ? sm.m[t] : -INFINITY;
            a.part_ml[pidx * 2 * kHG + kHG + t] = sm.l[t];
        }
    }
}

// Merge of the S partial softmaxes of 4 heads of one (sequence, head group):
// block of 256 threads, thread t -> head t / 64 of the four, dims
// (t % 64) * 8 .. + 7, so a wave reads one head's 2 KB row contiguously.
// The partial outputs of two splits are loaded together with their (m, l),
// so the common two-split case costs one round trip to memory.
constexpr int kMergeHeads = 4;
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a)
{
    const int HG = a.heads / kHG;
    constexpr int kQuarters = kHG / kMergeHeads;
    const int bh = blockIdx.x / kQuarters, b = bh / HG, hg = bh % HG;
    const int t = threadIdx.x, h = (blockIdx.x % kQuarters) * kMergeHeads + t / 64, d0 = (t % 64) * 8;
    const size_t p0 = ((size_t)b * HG + hg) * a.splits;
    float M = -INFINITY, L = 0.f;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // splits two at a time, with a running maximum (one pass when S = 2)
    for (int s0 = 0; s0 < a.splits; s0 += 2) {
        float4 x[2][2];
        float ms[2], ls[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = s0 + j < a.splits ? s0 + j : s0;
            ms[j] = a.part_ml[(p0 + s) * 2 * kHG + h];
            ls[j] = a.part_ml[(p0 + s) * 2 * kHG + kHG + h];
            const float4 *src = reinterpret_cast<const float4 *>(a.part_o + ((p0 + s) * kHG + h) * kDv + d0);
            x[j][0] = src[0];
            x[j][1] = src[1];
        }
        if (s0 + 1 >= a.splits) ms[1] = -INFINITY;
        const float Mn = fmaxf(M, fmaxf(ms[0], ms[1]));
        if (Mn == -INFINITY) continue;                 // nothing in these splits yet
        const float r = exp2f(M - Mn);                 // 0 while M is -inf
        L *= r;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= r;
        M = Mn;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (ms[j] == -INFINITY) continue;
            const float f = exp2f(ms[j] - M);
            L += f * ls[j];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                acc[4 * i] = fmaf(f, x[j][i].x, acc[4 * i]);
                acc[4 * i + 1] = fmaf(f, x[j][i].y, acc[4 * i + 1]);
                acc[4 * i + 2] = fmaf(f, x[j][i].z, acc[4 * i + 2]);
                acc[4 * i + 3] = fmaf(f, x[j][i].w, acc[4 * i + 3]);
            }
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const size_t head = (size_t)b * a.heads + kHG * hg + h;
    float4 *dst = reinterpret_cast<float4 *>(a.out + head * kDv + d0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        dst[i] = make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
    if (a.lse && (t & 63) == 0)
        a.lse[head] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

AttnPlan attn_plan(const cskv_cache &c, int heads, int k, int window)
{
    // Blocks of 8 waves, one per CU (the staging takes most of the LDS).  A
    // split takes per_sparse entry chunks and per_win window chunks; in the
    // kind-pure layout the entry splits come first and each split holds one
    // kind, in the mixed layout split i holds entry chunks and window chunks
    // both (one softmax state across the two loops).  The layout and split
    // sizes are chosen from a rough cost per block -- setup, then per chunk
    // a fixed cost about twice as high for 128 entries as for 64 window rows
    // -- times the rounds of 256 blocks, plus the merge when splitting.
    AttnPlan p;
    p.n_sparse = (k + kSK - 1) / kSK;
    p.n_win = (window + kWK - 1) / kWK;
    const int units = c.batch * (heads / kHG);
    double best = 1e300;
    p.per_sparse = p.n_sparse;
    p.per_win = p.n_win;
    p.win_split0 = 1;
    for (int mixed = 0; mixed < 2; ++mixed)
        for (int ps = 1; ps <= p.n_sparse && ps <= kMaxSplitChunks; ++ps)
            for (int pw = 1; pw <= p.n_win && pw <= kMaxSplitChunks; ++pw) {
                if (mixed && ps + pw > kMaxSplitChunks) continue;
                const int ss = (p.n_sparse + ps - 1) / ps, sw = (p.n_win + pw - 1) / pw;
                const int splits = mixed ? (ss > sw ? ss : sw) : ss + sw;
                const double rounds = ceil((double)units * splits / 256.0);
                const double chain = mixed ? 2.0 * ps + pw + 0.5 : fmax(2.0 * ps, 1.0 * pw);
                const double cost = rounds * (3.0 + chain) + (splits > 1 ? 4.0 : 0.0);
                if (cost < best - 1e-9) {
                    best = cost;
                    p.per_sparse = ps;
                    p.per_win = pw;
                    p.win_split0 = mixed ? 0 : ss;
                    p.splits = splits;
                }
            }
    const size_t parts = (size_t)units * p.splits;
    p.ws_bytes = p.splits > 1 ? parts * kHG * (kDv + 2) * sizeof(float) + 256 : 0;
    return p;
}

hipError_t launch_sparse_attn(const cskv_cache &c, const float *q, int heads, const int32_t *idx,
                              int k, const uint16_t *swa, int window, const int32_t *swa_len,
                              float scale, float *out, float *lse, void *ws, hipStream_t s)
{
    const AttnPlan p = attn_plan(c, heads, k, window);
    const int hg = heads / kHG;
    const size_t units = (size_t)c.batch * hg * p.splits;
    float *part_o = p.splits > 1 ? static_cast<float *>(ws) : nullptr;
    float *part_ml = p.splits > 1 ? part_o + units * kHG * kDv : nullptr;
    AttnArgs a{c, q, idx, swa, swa_len, out, lse, part_o, part_ml, heads, k, window,
               p.n_sparse, p.n_win, p.win_split0, p.per_sparse, p.per_win, p.splits,
               (float)((double)scale * 1.4426950408889634)};
    const int U = c.batch * p.splits;
    const unsigned blocks = (unsigned)(8 * hg * ((U + 7) / 8));
    const int vgs = c.v_group > 0 ? c.v_group : c.k_group;
    const TimedLaunch tl = timer_take(CSKV_KERNEL_ATTENTION);
    hipEvent_t stop_main = p.splits > 1 ? nullptr : tl.stop;
    auto attn = [&](auto kernel) { launch_kernel(kernel, dim3(blocks), dim3(kThreads), s, tl.start, stop_main, a); };
    auto pick = [&](auto w8) {
        constexpr bool W8 = decltype(w8)::value;
        if (c.k_format == CSKV_KV_MX16) {
            if (c.v_group > 0) attn(sparse_attn_kernel<16, true, 16, W8>);
            else attn(sparse_attn_kernel<16, false, 16, W8>);
            return;
        }
        if (c.v_group > 0) {
            if (c.k_group == 32) {
                if (vgs == 32) attn(sparse_attn_kernel<32, true, 32, W8>);
                else if (vgs == 64) attn(sparse_attn_kernel<64, true, 32, W8>);
                else attn(sparse_attn_kernel<128, true, 32, W8>);
            } else {
                if (vgs == 32) attn(sparse_attn_kernel<32, true, 64, W8>);
                else if (vgs == 64) attn(sparse_attn_kernel<64, true, 64, W8>);
                else attn(sparse_attn_kernel<128, true, 64, W8>);
            }
        } else {
            if (c.k_group == 32) attn(sparse_attn_kernel<32, false, 32, W8>);
            else attn(sparse_attn_kernel<64, false, 64, W8>);
        }
    };
    if (c.swa_format == CSKV_SWA_FP8) pick(std::true_type{});
    else pick(std::false_type{});
    if (p.splits > 1)
        launch_kernel(attn_merge_kernel, dim3((unsigned)(c.batch * hg * (kHG / kMergeHeads))), dim3(256), s,
                      nullptr, tl.stop, a);
    return hipGetLastError();
}

}  // namespace cskv
