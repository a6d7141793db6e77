// attention.hip -- gather + dequantise + one softmax over the selected
// compressed entries and the window rows, for all query heads of a sequence
// [P2 三、"突破四：滑动窗口和稀疏注意力" (sparse global branch + 128-token
// window); P2 三、"突破二：MLA，低秩压缩" (every head reads the same latent
// entry); P2 四、"P4 main KV" (FP4 is storage only; dequantise before use)].
//
// Work decomposition.  The keys of a sequence (the k selected entries, then
// the window rows) are cut into chunks of 32 and the chunks into S contiguous
// splits.  One block of 4 waves takes 16 query heads and one split; a second
// kernel merges the S partial softmaxes of each head by their log-sum-exp
// (skipped when S = 1).  The blocks that share a split's keys (one per head
// group) are numbered so that they land on the same XCD and read the gathered
// rows through one L2.
//
// Per chunk.  The gathered rows stay E2M1 codes in LDS: the key plane row-
// major (MFMA B operand of Q.K^T: 8 consecutive dims of one key = one 32-bit
// word of codes) and the value plane transposed to [dim][key] nibbles (B
// operand of P.V: 8 consecutive keys of one dim = one word).  Each operand
// word becomes 8 bf16 values with four hardware FP4 conversions; E2M1 values
// are exact in bf16.  Group scales stay fp32 outside the MFMA: per key group
// on the logits, folded into the probabilities per value group.  q and the
// scaled probabilities are each split into bf16 high and low parts, so the
// products carry about 16 significant bits.  Window rows are bf16 already and
// are staged row-major.  The softmax runs online in base 2 with fp32
// statistics.  The next chunk's HBM reads are issued before the current chunk
// is computed.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <math.h>

#include "device.hpp"
#include "launch.hpp"

namespace cskv {

namespace {

constexpr int kThreads = 512;    // 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kHG = 16;          // query heads per block (one MFMA row tile)
constexpr int kKC = 32;          // keys per chunk
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kSteps = kD / 32;  // 18 contraction steps of Q.K^T
constexpr int kParts = 4;        // the steps are shared by 4 waves per key tile
constexpr int kMaxPart = 5;      // steps per part: 5, 5, 4, 4
constexpr int kMaxKG = kD / 32;
constexpr int kMaxVG = kDv / 32;
constexpr int kCodeRow = kD / 2 + 16;     // 304 B: conflict-free 32-bit operand reads
constexpr int kVCodeRow = kDv / 2 + 16;   // 272 B
constexpr int kWinRow = kD + 8;           // 584 bf16 = 1168 B
constexpr int kMaxSplitChunks = 32;       // chunk indices a block keeps in LDS

__device__ __forceinline__ int part_begin(int p) { return p < 2 ? 5 * p : 10 + 4 * (p - 2); }

struct SparseStage {
    uint8_t kc[kKC][kCodeRow];            // key-plane codes, row-major
    uint8_t vc[kKC][kVCodeRow];           // value-plane codes (split planes only)
    uint32_t vt[kDv][kKC / 8];            // value codes transposed: [dim][8-key word]
};
struct WindowStage {
    uint16_t kr[kKC][kWinRow];            // window rows, bf16
};

struct AttnSmem {
    union {
        SparseStage sp;
        WindowStage win;
    } st;
    float ks[kKC][kMaxKG];                // key-plane scale per key and group (1: window)
    float vs[kKC][kMaxVG];                // value scale per key and value group
    float spart[kParts][kHG][kKC + 1];    // logits from the 4 parts of the contraction
    float p[kHG][kKC + 4];                // probabilities of the chunk
    float m[kHG], l[kHG], alpha[kHG];
    int32_t src[kMaxSplitChunks * kKC];   // entry index / window slot per key, -1 masked
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
    int n_sparse;       // chunks of selected entries
    int n_chunks;       // + chunks of window rows
    int splits, per_split;
    float scale_log2;   // softmax_scale * log2(e)
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

// hi/lo bf16 split of 8 floats: x = hi + lo + O(2^-17 |x|)
__device__ __forceinline__ void split8(const float *x, u32x4_t &hi, u32x4_t &lo)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h0 = bf16_bits_rne(x[2 * i]), h1 = bf16_bits_rne(x[2 * i + 1]);
        const uint32_t l0 = bf16_bits_rne(x[2 * i] - bf16_bits_to_f32(h0));
        const uint32_t l1 = bf16_bits_rne(x[2 * i + 1] - bf16_bits_to_f32(h1));
        hi[i] = h0 | (h1 << 16);
        lo[i] = l0 | (l1 << 16);
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

// Registers holding one chunk's HBM reads until they are written to LDS.
struct Prefetch {
    u32x4_t w[5];       // 16-byte pieces (sparse: key codes 0-1, value codes 2; window: 0-4)
    float sc[3];        // key scales 0-1, value scales 2
};

// VGS: the value group size in effect (the value plane's group, else the key
// plane's): 32, 64 or 128.
template <int VGS>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_kernel(AttnArgs a)
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
    const int c0 = split * a.per_split;
    const int c1 = min(a.n_chunks, c0 + a.per_split);

    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t E = entries_of(c.n_tokens, b, c.capacity);
    int64_t nswa = a.swa_len ? (int64_t)a.swa_len[b] : (int64_t)c.n_tokens[b];
    nswa = nswa < 0 ? 0 : (nswa > a.window ? a.window : nswa);

    const int kg = c.k_group, G = kD / kg;
    const bool split_v = c.v_group > 0;
    constexpr int VG = kDv / VGS;
    const float *vscales = split_v ? c.v_scales : c.k_scales;
    const int vscale_row = split_v ? VG : G;
    const size_t row0 = (size_t)b * c.capacity;

    // ---- key sources of every chunk of the split
    for (int i = t; i < (c1 - c0) * kKC; i += kThreads) {
        const int chunk = c0 + i / kKC, j = i % kKC;
        int32_t s = -1;
        if (chunk < a.n_sparse) {
            const int jj = chunk * kKC + j;
            const int32_t e = jj < a.k ? a.idx[(size_t)b * a.k + jj] : -1;
            s = (e >= 0 && e < E) ? e : -1;
        } else {
            const int64_t slot = (int64_t)(chunk - a.n_sparse) * kKC + j;
            s = slot < nswa ? (int32_t)slot : -1;
        }
        sm.src[i] = s;
    }
    if (t < kHG) { sm.m[t] = -1e30f; sm.l[t] = 0.f; }

    // ---- query operands: wave w takes key tile kt = w & 1 and contraction
    // steps [s0, s0 + ns) of part w >> 1; rows = heads of this group, hi + lo
    const int kt = w & 1, part = w >> 1;
    const int s0 = part_begin(part), ns = part_begin(part + 1) - s0;
    u32x4_t qhi[kMaxPart], qlo[kMaxPart];
    {
        const float *qrow = a.q + ((size_t)b * a.heads + kHG * hg + col) * kD + 8 * grp;
#pragma unroll
        for (int s = 0; s < kMaxPart; ++s) {
            const int step = s < ns ? s0 + s : s0;
            const float4 x0 = *reinterpret_cast<const float4 *>(qrow + 32 * step);
            const float4 x1 = *reinterpret_cast<const float4 *>(qrow + 32 * step + 4);
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            split8(x, qhi[s], qlo[s]);
        }
    }
    f32x4_t o[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    // ---- HBM reads of one chunk into registers
    auto fetch = [&](int chunk, Prefetch &pf) {
        const int32_t *src = sm.src + (chunk - c0) * kKC;
        if (chunk < a.n_sparse) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {                  // 32 keys x 18 pieces of key codes
                const int task = t + kThreads * i, j = task / 18, piece = task % 18;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (task < kKC * 18 && src[j] >= 0)
                    v = *reinterpret_cast<const u32x4_t *>(c.k_codes + (row0 + src[j]) * (kD / 2) + 16 * piece);
                pf.w[i] = v;
            }
            if (split_v) {                                 // 32 keys x 16 pieces of value codes
                const int j = t / 16, piece = t % 16;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (src[j] >= 0)
                    v = *reinterpret_cast<const u32x4_t *>(c.v_codes + (row0 + src[j]) * (kDv / 2) + 16 * piece);
                pf.w[2] = v;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {                  // key scales: 32 x G
                const int task = t + kThreads * i, j = task / G, g = task % G;
                pf.sc[i] = (task < kKC * G && src[j] >= 0) ? c.k_scales[(row0 + src[j]) * G + g] : 0.f;
            }
            {                                              // value scales: 32 x VG
                const int j = t / VG, g = t % VG;
                pf.sc[2] = (t < kKC * VG && src[j] >= 0) ? vscales[(row0 + src[j]) * vscale_row + g] : 0.f;
            }
        } else {
            const uint16_t *ring = a.swa + (size_t)b * a.window * kD;
#pragma unroll
            for (int i = 0; i < 5; ++i) {                  // 32 rows x 72 pieces
                const int task = t + kThreads * i, j = task / 72, piece = task % 72;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (task < kKC * 72 && src[j] >= 0)
                    v = *reinterpret_cast<const u32x4_t *>(ring + (size_t)src[j] * kD + 8 * piece);
                pf.w[i] = v;
            }
        }
    };

    auto store = [&](int chunk, const Prefetch &pf) {
        if (chunk < a.n_sparse) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int task = t + kThreads * i, j = task / 18, piece = task % 18;
                if (task < kKC * 18) *reinterpret_cast<u32x4_t *>(&sm.st.sp.kc[j][16 * piece]) = pf.w[i];
            }
            if (split_v) *reinterpret_cast<u32x4_t *>(&sm.st.sp.vc[t / 16][16 * (t % 16)]) = pf.w[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int task = t + kThreads * i;
                if (task < kKC * G) sm.ks[task / G][task % G] = pf.sc[i];
            }
            if (t < kKC * VG) sm.vs[t / VG][t % VG] = pf.sc[2];
        } else {
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int task = t + kThreads * i, j = task / 72, piece = task % 72;
                if (task < kKC * 72) *reinterpret_cast<u32x4_t *>(&sm.st.win.kr[j][8 * piece]) = pf.w[i];
            }
            for (int i = t; i < kKC * kMaxKG; i += kThreads) sm.ks[i / kMaxKG][i % kMaxKG] = 1.f;
            for (int i = t; i < kKC * kMaxVG; i += kThreads) sm.vs[i / kMaxVG][i % kMaxVG] = 1.f;
        }
    };

    Prefetch pf;
    if (c0 < c1) fetch(c0, pf);
    for (int chunk = c0; chunk < c1; ++chunk) {
        const bool sparse = chunk < a.n_sparse;
        const int32_t *src = sm.src + (chunk - c0) * kKC;
        __syncthreads();                                   // previous chunk fully consumed
        store(chunk, pf);
        __syncthreads();
        if (chunk + 1 < c1) fetch(chunk + 1, pf);

        // ---- value codes transposed to [dim][key word]: task = (key octet, dim octet)
        if (sparse) {
            if (t < 256) {
                const int oct = t & 3, doct = t >> 2;      // 4 key octets x 64 dim octets
                uint32_t in[8], outw[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    in[j] = split_v ? *reinterpret_cast<const uint32_t *>(&sm.st.sp.vc[8 * oct + j][4 * doct])
                                    : *reinterpret_cast<const uint32_t *>(&sm.st.sp.kc[8 * oct + j][4 * doct]);
                transpose_nibbles(in, outw);
#pragma unroll
                for (int d = 0; d < 8; ++d) sm.st.sp.vt[8 * doct + d][oct] = outw[d];
            }
            __syncthreads();
        }

        // ---- logits of key tile kt over this wave's contraction steps
        {
            const int j = 16 * kt + col;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kMaxPart; ++s) {
                if (s < ns) {
                    const int step = s0 + s;
                    u32x4_t kb;
                    if (sparse) kb = fp4x8_to_bf16x8(*reinterpret_cast<const uint32_t *>(&sm.st.sp.kc[j][16 * step + 4 * grp]));
                    else kb = lds16(&sm.st.win.kr[j][32 * step + 8 * grp]);
                    f32x4_t pr = {0.f, 0.f, 0.f, 0.f};
                    pr = mfma16x16x32(qhi[s], kb, pr);
                    pr = mfma16x16x32(qlo[s], kb, pr);
                    const float sc = sm.ks[j][(32 * step) / kg];
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, pr[v], acc[v]);
                }
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.spart[part][4 * grp + v][j] = acc[v];
        }
        __syncthreads();

        // ---- online softmax: thread t -> head t / 32, key t % 32
        {
            const int h = t >> 5, j = t & 31;
            const float sum4 = (sm.spart[0][h][j] + sm.spart[1][h][j]) + (sm.spart[2][h][j] + sm.spart[3][h][j]);
            const float sv = src[j] >= 0 ? sum4 * a.scale_log2 : -INFINITY;
            float mx = sv;
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_old = sm.m[h];
            const float m_new = fmaxf(m_old, mx);
            const float pj = exp2f(sv - m_new);
            float sum = pj;
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
            sm.p[h][j] = pj;
            if (j == 0) {
                const float al = exp2f(m_old - m_new);
                sm.alpha[h] = al;
                sm.m[h] = m_new;
                sm.l[h] = sm.l[h] * al + sum;
            }
        }
        __syncthreads();

        // ---- P.V: wave w owns value dims [64 w, 64 w + 64) = 4 tiles of 16
        {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float al = sm.alpha[4 * grp + v];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) o[nt][v] *= al;
            }
            constexpr int kGroupsHere = VGS >= 64 ? 1 : 64 / VGS;   // value groups per wave
            constexpr int kTilesPerGroup = 4 / kGroupsHere;
#pragma unroll
            for (int gi = 0; gi < kGroupsHere; ++gi) {
                const int gv = (64 * w) / VGS + gi;
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = sm.p[col][8 * grp + i] * sm.vs[8 * grp + i][gv];
                u32x4_t phi, plo;
                split8(pv, phi, plo);
#pragma unroll
                for (int tt = 0; tt < kTilesPerGroup; ++tt) {
                    const int nt = gi * kTilesPerGroup + tt;
                    const int dim = 64 * w + 16 * nt + col;
                    u32x4_t vb;
                    if (sparse) {
                        vb = fp4x8_to_bf16x8(sm.st.sp.vt[dim][grp]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            vb[i] = (uint32_t)sm.st.win.kr[8 * grp + 2 * i][dim] |
                                    ((uint32_t)sm.st.win.kr[8 * grp + 2 * i + 1][dim] << 16);
                    }
                    o[nt] = mfma16x16x32(phi, vb, o[nt]);
                    o[nt] = mfma16x16x32(plo, vb, o[nt]);
                }
            }
        }
    }
    __syncthreads();

    // ---- results: final (one split) or partial (merged by attn_merge_kernel)
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

// Merge of the S partial softmaxes of one (sequence, head group): block of
// 256 threads, thread t -> head t / 16, dims (t % 16) * 32 .. + 31.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a)
{
    const int HG = a.heads / kHG;
    const int bh = blockIdx.x, b = bh / HG, hg = bh % HG;
    const int t = threadIdx.x, h = t >> 4, d0 = (t & 15) * 32;
    const size_t p0 = ((size_t)b * HG + hg) * a.splits;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(p0 + s) * 2 * kHG + h]);
    float L = 0.f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    if (M > -INFINITY) {
        for (int s = 0; s < a.splits; ++s) {
            const float ms = a.part_ml[(p0 + s) * 2 * kHG + h];
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            L += f * a.part_ml[(p0 + s) * 2 * kHG + kHG + h];
            const float4 *src = reinterpret_cast<const float4 *>(a.part_o + ((p0 + s) * kHG + h) * kDv + d0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 x = src[i];
                acc[4 * i] = fmaf(f, x.x, acc[4 * i]);
                acc[4 * i + 1] = fmaf(f, x.y, acc[4 * i + 1]);
                acc[4 * i + 2] = fmaf(f, x.z, acc[4 * i + 2]);
                acc[4 * i + 3] = fmaf(f, x.w, acc[4 * i + 3]);
            }
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const size_t head = (size_t)b * a.heads + kHG * hg + h;
    float4 *dst = reinterpret_cast<float4 *>(a.out + head * kDv + d0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dst[i] = make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
    if (a.lse && (t & 15) == 0)
        a.lse[head] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

AttnPlan attn_plan(const cskv_cache &c, int heads, int k, int window)
{
    AttnPlan p;
    p.n_sparse = (k + kKC - 1) / kKC;
    p.n_chunks = p.n_sparse + (window + kKC - 1) / kKC;
    const int hg = heads / kHG;
    // about one block (8 waves) per CU
    int splits = (256 + c.batch * hg - 1) / (c.batch * hg);
    splits = splits < 1 ? 1 : (splits > p.n_chunks ? p.n_chunks : splits);
    p.per_split = (p.n_chunks + splits - 1) / splits;
    if (p.per_split > kMaxSplitChunks) p.per_split = kMaxSplitChunks;
    p.splits = (p.n_chunks + p.per_split - 1) / p.per_split;
    const size_t units = (size_t)c.batch * hg * p.splits;
    p.ws_bytes = p.splits > 1 ? units * kHG * (kDv + 2) * sizeof(float) + 256 : 0;
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
               p.n_sparse, p.n_chunks, p.splits, p.per_split,
               (float)((double)scale * 1.4426950408889634)};
    const int U = c.batch * p.splits;
    const unsigned blocks = (unsigned)(8 * hg * ((U + 7) / 8));
    const int vgs = c.v_group > 0 ? c.v_group : c.k_group;
    timer_before(CSKV_KERNEL_ATTENTION, s);
    if (vgs == 32) sparse_attn_kernel<32><<<blocks, kThreads, 0, s>>>(a);
    else if (vgs == 64) sparse_attn_kernel<64><<<blocks, kThreads, 0, s>>>(a);
    else sparse_attn_kernel<128><<<blocks, kThreads, 0, s>>>(a);
    if (p.splits > 1) attn_merge_kernel<<<(unsigned)(c.batch * hg), 256, 0, s>>>(a);
    timer_after(CSKV_KERNEL_ATTENTION, s);
    return hipGetLastError();
}

}  // namespace cskv
