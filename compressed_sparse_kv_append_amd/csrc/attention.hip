// attention.hip -- gather + dequantise + one softmax over the selected
// compressed entries and the window rows, for all query heads of a sequence
// [P2 三、"突破四：滑动窗口和稀疏注意力" (sparse global branch + 128-token
// window); P2 三、"突破二：MLA，低秩压缩" (every head reads the same latent
// entry); P2 四、"P4 main KV" (FP4 is storage only; dequantise before use)].
//
// Block = one sequence x 16 query heads, 4 waves.  Keys are processed in
// chunks of 32: the gathered E2M1 codes are expanded into LDS as bf16 values,
// which is exact (every E2M1 value has at most 2 significant bits); the group
// scales stay fp32 and are applied outside the MFMA: per key group for the
// logits, folded into the probabilities per value group for P.V.  q and the
// scaled probabilities are each split into a bf16 high and low part, so the
// products carry ~16 significant bits and the fp32 accumulation dominates
// the error.  The softmax runs online in base 2 with fp32 statistics.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <math.h>

#include "device.hpp"
#include "launch.hpp"

namespace cskv {
namespace {

constexpr int kThreads = 256;
constexpr int kHG = 16;        // query heads per block (one MFMA row tile)
constexpr int kKC = 32;        // keys per chunk (one MFMA contraction step of P.V)
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kRow = 584;      // padded bf16 row: 1168 B keeps 16-row operand reads conflict-free
constexpr int kVtRow = 40;     // padded transposed value row: 32 keys + 8
constexpr int kMaxKG = kD / 32;
constexpr int kMaxVG = kDv / 32;

struct AttnSmem {
    uint16_t qhi[kHG][kRow];
    uint16_t qlo[kHG][kRow];
    uint16_t krow[kKC][kRow];       // keys of the chunk, bf16 (E2M1 values or window rows)
    uint16_t vt[kDv][kVtRow];       // values of the chunk, transposed: [dim][key]
    float ks[kKC][kMaxKG];          // key-plane scale per key and group (1 for window rows)
    float vs[kKC][kMaxVG];          // value scale per key and value group
    float spart[2][kHG][kKC + 1];   // logits from the two halves of the groups
    float p[kHG][kKC + 4];          // probabilities of the chunk
    float m[kHG], l[kHG], alpha[kHG];
    int32_t src[kKC];               // entry index / window slot of each key, -1 = masked
};

struct AttnArgs {
    cskv_cache c;
    const float *q;
    const int32_t *idx;
    const uint16_t *swa;
    const int32_t *swa_len;
    float *out;
    float *lse;
    int heads, k, window;
    float scale_log2;   // softmax_scale * log2(e)
};

__device__ __forceinline__ u32x4_t lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4_t *>(p); }

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

__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(AttnArgs a)
{
    __shared__ AttnSmem sm;
    const cskv_cache &c = a.c;
    const int hg = blockIdx.x, b = blockIdx.y;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int64_t E = entries_of(c.n_tokens, b, c.capacity);
    int64_t nswa = a.swa_len ? (int64_t)a.swa_len[b] : (int64_t)c.n_tokens[b];
    nswa = nswa < 0 ? 0 : (nswa > a.window ? a.window : nswa);

    const int kg = c.k_group, G = kD / kg, gsteps = kg / 32;
    const bool split_v = c.v_group > 0;
    const int vg = split_v ? c.v_group : kg, VG = kDv / vg;
    const uint8_t *vcodes = split_v ? c.v_codes : c.k_codes;
    const float *vscales = split_v ? c.v_scales : c.k_scales;
    const int vscale_row = split_v ? VG : G;       // scales per entry in that plane
    const int vrow_bytes = split_v ? kDv / 2 : kD / 2;

    // query rows of this head group, split into bf16 hi + lo
    for (int i = t; i < kHG * kD; i += kThreads) {
        const int h = i / kD, d = i % kD;
        const float x = a.q[((size_t)b * a.heads + kHG * hg + h) * kD + d];
        const uint32_t hi = bf16_bits_rne(x);
        sm.qhi[h][d] = (uint16_t)hi;
        sm.qlo[h][d] = (uint16_t)bf16_bits_rne(x - bf16_bits_to_f32(hi));
    }
    if (t < kHG) { sm.m[t] = -1e30f; sm.l[t] = 0.f; }
    f32x4_t o[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int n_sparse = (a.k + kKC - 1) / kKC;
    const int n_chunks = n_sparse + (int)((nswa + kKC - 1) / kKC);
    for (int chunk = 0; chunk < n_chunks; ++chunk) {
        const bool from_swa = chunk >= n_sparse;
        __syncthreads();                                   // previous chunk consumed
        if (t < kKC) {
            int32_t s = -1;
            if (!from_swa) {
                const int j = chunk * kKC + t;
                const int32_t e = j < a.k ? a.idx[(size_t)b * a.k + j] : -1;
                s = (e >= 0 && e < E) ? e : -1;
            } else {
                const int64_t slot = (int64_t)(chunk - n_sparse) * kKC + t;
                s = slot < nswa ? (int32_t)slot : -1;
            }
            sm.src[t] = s;
        }
        __syncthreads();

        // ---- stage keys (row-major) and values (transposed) of the chunk
        if (!from_swa) {
            for (int task = t; task < kKC * (kD / 16); task += kThreads) {
                const int j = task / (kD / 16), piece = task % (kD / 16);
                const int32_t e = sm.src[j];
                uint2 cw = make_uint2(0u, 0u);
                if (e >= 0)
                    cw = *reinterpret_cast<const uint2 *>(
                        c.k_codes + ((size_t)b * c.capacity + e) * (kD / 2) + piece * 8);
                *reinterpret_cast<u32x4_t *>(&sm.krow[j][piece * 16]) = e2m1x8_to_bf16x8(cw.x);
                *reinterpret_cast<u32x4_t *>(&sm.krow[j][piece * 16 + 8]) = e2m1x8_to_bf16x8(cw.y);
            }
            for (int task = t; task < kKC * G; task += kThreads) {
                const int j = task / G, g = task % G;
                const int32_t e = sm.src[j];
                sm.ks[j][g] = e >= 0 ? c.k_scales[((size_t)b * c.capacity + e) * G + g] : 0.f;
            }
            for (int task = t; task < kKC * VG; task += kThreads) {
                const int j = task / VG, g = task % VG;
                const int32_t e = sm.src[j];
                sm.vs[j][g] = e >= 0 ? vscales[((size_t)b * c.capacity + e) * vscale_row + g] : 0.f;
            }
            // transposed values: task = (code byte c2 -> dims 2c2, 2c2+1) x (octet of keys)
            for (int task = t; task < (kDv / 2) * (kKC / 8); task += kThreads) {
                const int c2 = task % (kDv / 2), oct = task / (kDv / 2);
                uint32_t lo_w[4], hi_w[4];
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    uint32_t v2[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int32_t e = sm.src[8 * oct + jj + x];
                        v2[x] = e >= 0 ? vcodes[((size_t)b * c.capacity + e) * vrow_bytes + c2] : 0u;
                    }
                    lo_w[jj / 2] = e2m1_to_bf16_bits(v2[0] & 0xFu) | (e2m1_to_bf16_bits(v2[1] & 0xFu) << 16);
                    hi_w[jj / 2] = e2m1_to_bf16_bits(v2[0] >> 4) | (e2m1_to_bf16_bits(v2[1] >> 4) << 16);
                }
                *reinterpret_cast<u32x4_t *>(&sm.vt[2 * c2][8 * oct]) = u32x4_t{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
                *reinterpret_cast<u32x4_t *>(&sm.vt[2 * c2 + 1][8 * oct]) = u32x4_t{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
            }
        } else {
            const uint16_t *ring = a.swa + (size_t)b * a.window * kD;
            for (int task = t; task < kKC * (kD / 8); task += kThreads) {
                const int j = task / (kD / 8), piece = task % (kD / 8);
                const int32_t s = sm.src[j];
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (s >= 0) v = *reinterpret_cast<const u32x4_t *>(ring + (size_t)s * kD + piece * 8);
                *reinterpret_cast<u32x4_t *>(&sm.krow[j][piece * 8]) = v;
            }
            for (int task = t; task < kKC * kMaxKG; task += kThreads) sm.ks[task / kMaxKG][task % kMaxKG] = 1.f;
            for (int task = t; task < kKC * kMaxVG; task += kThreads) sm.vs[task / kMaxVG][task % kMaxVG] = 1.f;
            for (int task = t; task < (kDv / 2) * (kKC / 8); task += kThreads) {
                const int c2 = task % (kDv / 2), oct = task / (kDv / 2);
                uint32_t lo_w[4], hi_w[4];
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    uint32_t v2[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int32_t s = sm.src[8 * oct + jj + x];
                        v2[x] = s >= 0 ? *reinterpret_cast<const uint32_t *>(ring + (size_t)s * kD + 2 * c2) : 0u;
                    }
                    lo_w[jj / 2] = (v2[0] & 0xFFFFu) | (v2[1] << 16);
                    hi_w[jj / 2] = (v2[0] >> 16) | (v2[1] & 0xFFFF0000u);
                }
                *reinterpret_cast<u32x4_t *>(&sm.vt[2 * c2][8 * oct]) = u32x4_t{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
                *reinterpret_cast<u32x4_t *>(&sm.vt[2 * c2 + 1][8 * oct]) = u32x4_t{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
            }
        }
        __syncthreads();

        // ---- logits: wave w takes key tile (w & 1) and half (w >> 1) of the groups
        {
            const int ntile = w & 1, half = w >> 1;
            const int g0 = half ? G / 2 : 0, g1 = half ? G : G / 2;
            const int j = 16 * ntile + (lane & 15);
            const int qh = lane & 15, sub = 8 * (lane >> 4);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int g = g0; g < g1; ++g) {
                f32x4_t part = {0.f, 0.f, 0.f, 0.f};
                for (int st = 0; st < gsteps; ++st) {
                    const int d0 = 32 * (g * gsteps + st) + sub;
                    const u32x4_t kb = lds16(&sm.krow[j][d0]);
                    part = mfma16x16x32(lds16(&sm.qhi[qh][d0]), kb, part);
                    part = mfma16x16x32(lds16(&sm.qlo[qh][d0]), kb, part);
                }
                const float sc = sm.ks[j][g];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, part[v], acc[v]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.spart[half][4 * (lane >> 4) + v][j] = acc[v];
        }
        __syncthreads();

        // ---- online softmax: thread t -> head t/16, keys 2*(t%16), +1
        {
            const int h = t >> 4, j0 = 2 * (t & 15);
            float s[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int j = j0 + i;
                s[i] = sm.src[j] >= 0 ? (sm.spart[0][h][j] + sm.spart[1][h][j]) * a.scale_log2 : -INFINITY;
            }
            float mx = fmaxf(s[0], s[1]);
            for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_old = sm.m[h];
            const float m_new = fmaxf(m_old, mx);
            const float p0 = exp2f(s[0] - m_new), p1 = exp2f(s[1] - m_new);
            float sum = p0 + p1;
            for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
            sm.p[h][j0] = p0;
            sm.p[h][j0 + 1] = p1;
            if ((t & 15) == 0) {
                const float al = exp2f(m_old - m_new);
                sm.alpha[h] = al;
                sm.m[h] = m_new;
                sm.l[h] = sm.l[h] * al + sum;
            }
        }
        __syncthreads();

        // ---- P.V: wave w owns value dims [128w, 128w+128) = 8 tiles of 16
        {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float al = sm.alpha[4 * (lane >> 4) + v];
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) o[nt][v] *= al;
            }
            const int ph = lane & 15, sub = 8 * (lane >> 4);
            const int groups_here = 128 / vg < 1 ? 1 : 128 / vg;
            const int tiles_per_group = 8 / groups_here;
            for (int gi = 0; gi < groups_here; ++gi) {
                const int gv = (128 * w) / vg + gi;
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = sm.p[ph][sub + i] * sm.vs[sub + i][gv];
                u32x4_t phi, plo;
                split8(pv, phi, plo);
                for (int tt = 0; tt < tiles_per_group; ++tt) {
                    const int nt = gi * tiles_per_group + tt;
                    const u32x4_t vb = lds16(&sm.vt[128 * w + 16 * nt + (lane & 15)][sub]);
                    o[nt] = mfma16x16x32(phi, vb, o[nt]);
                    o[nt] = mfma16x16x32(plo, vb, o[nt]);
                }
            }
        }
    }
    __syncthreads();

    // ---- normalise and write
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int h = 4 * (lane >> 4) + v;
        const float l = sm.l[h];
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float *orow = a.out + ((size_t)b * a.heads + kHG * hg + h) * kDv + 128 * w + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = o[nt][v] * inv;
    }
    if (a.lse && t < kHG) {
        const float l = sm.l[t];
        a.lse[(size_t)b * a.heads + kHG * hg + t] =
            l > 0.f ? (sm.m[t] + log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace

hipError_t launch_sparse_attn(const cskv_cache &c, const float *q, int heads, const int32_t *idx,
                              int k, const uint16_t *swa, int window, const int32_t *swa_len,
                              float scale, float *out, float *lse, hipStream_t s)
{
    AttnArgs a{c, q, idx, swa, swa_len, out, lse, heads, k, window,
               (float)((double)scale * 1.4426950408889634)};
    dim3 grid((unsigned)(heads / kHG), (unsigned)c.batch);
    timer_before(CSKV_KERNEL_ATTENTION, s);
    sparse_attn_kernel<<<grid, kThreads, 0, s>>>(a);
    timer_after(CSKV_KERNEL_ATTENTION, s);
    return hipGetLastError();
}

}  // namespace cskv
