// append.hip -- cache append: 2->1 compression, group FP4 quantisation and
// packing, pending-token bookkeeping, and the sliding-window rows.
//
// Sources cited as [P1]/[P2] (page title, then the section):
//   P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <type_traits>

#include "append_dev.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {
namespace {

// One block per input row.  A block whose row completes an entry quantises
// that entry (compressor mode: from the compressor's output; entries mode:
// the row itself) and writes its codes, scales and indexer key.  kFinalize
// (one row per sequence): the block then also finalises its sequence and
// writes the row's window entry when a window ring is given.  kHead (a
// decode step, one row per sequence, compressor mode): the block writes only
// the entry's indexer key and records its cache row in a.slots (-1: none);
// the entry itself is compressed and quantised later (quantize_main_512),
// by kernels that run after this one and read the record, so the token
// counts can advance here.
template <bool kCompress, bool kFinalize, bool kHead = false>
__global__ __launch_bounds__(kAppendThreads) void quantize_kernel(AppendArgs a)
{
    static_assert(!kHead || (kCompress && kFinalize), "the head of a one-row compressor append");
    __shared__ float wave_max[kAppendThreads / kWave];
    const cskv_cache &c = a.c;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    // every load of the block is issued before any is waited for (the
    // entry row of a row that completes none is read and dropped)
    const int b0 = seq_of_row(a.cu_new, c.batch, (int)r);
    const int64_t p = c.n_tokens[b0];
    const float ev = kHead ? 0.f : kCompress ? a.ent[(size_t)r * kDim + t] : a.tokens[(size_t)r * kDim + t];
    const uint16_t key_t = a.idx_rows[(size_t)r * c.idx_dim + (t < c.idx_dim ? t : 0)];
    const float xw = kFinalize && a.swa_ring ? a.swa_rows[(size_t)r * kDim + t] : 0.f;
    const RowInfo ri = row_info<kCompress>(a, r, b0, p);
    int64_t rec = -1;
    if (ri.entry >= 0) {
        const int64_t slot = plane_row(c, ri.b, ri.entry);
        if (slot >= 0) {
            if (kHead) store_idx_key(a, t, (size_t)slot, key_t);
            else quantize_entry(a, ev, t, (size_t)slot, key_t, wave_max);
            rec = slot;
        } else if (t == 0) {
            atomicOr(c.status, CSKV_STATUS_BAD_PAGE);
        }
    }
    if (kHead && t == 0) a.slots[r] = rec;
    if (kFinalize) {
        const int b = (int)r;
        __syncthreads();                            // every thread has read n_tokens[b]
        const int64_t end = finalize_seq<kCompress>(a, b, p, t, kAppendThreads);
        if (a.swa_ring && end >= 1) {
            const int64_t pos = end - 1;            // the position of this row's token
            const size_t row = (size_t)b * a.swa_window + (size_t)(pos % a.swa_window);
            const float x = xw;
            if (c.swa_format == CSKV_SWA_FP8)
                reinterpret_cast<uint8_t *>(a.swa_ring)[row * kDim + t] = (uint8_t)e4m3_bits(x);
            else
                a.swa_ring[row * kDim + t] = (uint16_t)bf16_bits_rne(x);
        }
    }
}

// One wave per sequence, after the quantiser (several rows per sequence).
template <bool kCompress>
__global__ __launch_bounds__(kWave) void append_finalize_kernel(AppendArgs a)
{
    const int b = blockIdx.x;
    (void)finalize_seq<kCompress>(a, b, a.c.n_tokens[b], threadIdx.x, kWave);
}

struct SwaArgs {
    uint16_t *ring;
    int batch, window, dim;
    const float *rows;
    const int32_t *cu_new;
    const int32_t *end_pos;
    int64_t total_new;
};

// One wave per row: fp32 -> bf16 (nearest even) or E4M3 (FP8) into ring slot
// pos % window when the row is among the last `window` positions.
template <bool FP8>
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
    const size_t slot = (size_t)b * a.window + (size_t)(pos % a.window);
    if (FP8) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.ring) + slot * a.dim);
        for (int i = t; i < a.dim / 4; i += kWave) {
            const float4 x = src[i];
            dst[i] = e4m3_bits(x.x) | (e4m3_bits(x.y) << 8) | (e4m3_bits(x.z) << 16) | (e4m3_bits(x.w) << 24);
        }
    } else {
        uint2 *dst = reinterpret_cast<uint2 *>(a.ring + slot * a.dim);
        for (int i = t; i < a.dim / 4; i += kWave) {
            const float4 x = src[i];
            uint2 o;
            o.x = bf16_bits_rne(x.x) | (bf16_bits_rne(x.y) << 16);
            o.y = bf16_bits_rne(x.z) | (bf16_bits_rne(x.w) << 16);
            dst[i] = o;
        }
    }
}

// ---------------------------------------------------------- large appends
//
// An append of many rows (a prefill chunk) runs the same compressor order
// as a tiled SIMT product.  A plan kernel first lists the rows that complete
// an entry; the compressor then gives each block a tile of 64 listed entries
// x 32 output channels and cuts each output's 64 term blocks into eight runs
// of 8, one per wave.  A run of 8 consecutive blocks is exactly one level-3
// node of the pairwise tree, so a wave folds its blocks and adds their sums
// in tree order, and the block joins the eight run sums as the tree's top
// three levels: ((r0 + r1) + (r2 + r3)) + ((r4 + r5) + (r6 + r7)).  The
// result equals the wave-per-output kernel's bit for bit.

constexpr int kPlanThreads = 1024;
constexpr int kTcRows = 64;                        // listed entries per block
constexpr int kTcCh = 32;                          // output channels per block
constexpr int kTcRuns = 8;                         // waves; run w = term blocks 8w .. 8w + 7
constexpr int kTcThreads = kTcRuns * kWave;
constexpr int kTcRunBlocks = (2 * kDim / kCompTerms) / kTcRuns;   // 8 term blocks per run
constexpr int kTcChTiles = kDim / kTcCh;           // 18
constexpr int kTcOpFloats = kCompTerms * (kTcRows + kTcCh);        // one wave's operands
constexpr int kTcLdsFloats = kTcRuns * (kTcOpFloats + kTcRows * kTcCh);   // operands, then run sums
static_assert(kTcRunBlocks == 8 && kTcRows == 64 && kTcCh == 32, "tile shape assumed below");
// Entries the plan can list: each sequence of m rows completes at most
// ceil(m / 2), so at most (total_new + batch) / 2 in all, and never more
// than total_new.
__host__ __device__ inline int64_t plan_bound(int64_t total_new, int batch)
{
    const int64_t b = (total_new + batch + 1) / 2;
    return b < total_new ? b : total_new;
}

// One block.  For every sequence (1024 at a time): the entries its rows
// complete (none when row_info would reject the sequence), an exclusive
// prefix over sequences, then one plan record per completed entry in
// sequence order: {input row, sequence, row of x_even (-1: pending), entry}.
// count receives the number of records.
__global__ __launch_bounds__(kPlanThreads) void compress_plan_kernel(AppendArgs a, int4 *plan, int32_t *count)
{
    __shared__ int s_off[kPlanThreads], s_row0[kPlanThreads], s_p[kPlanThreads];
    __shared__ int s_wave[kPlanThreads / kWave];
    const cskv_cache &c = a.c;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    int carry = 0;
    for (int b0 = 0; b0 < c.batch; b0 += kPlanThreads) {
        const int b = b0 + t;
        int cnt = 0, row0 = 0, p = 0;
        if (b < c.batch) {
            row0 = a.cu_new ? a.cu_new[b] : b;
            const int64_t m = a.cu_new ? (int64_t)a.cu_new[b + 1] - row0 : 1;
            p = c.n_tokens[b];
            if (p >= 0 && rows_ok(row0, m, a.total_new) && (p + m) / 2 <= c.capacity)
                cnt = (int)((p + m) / 2 - p / 2);
        }
        int x = cnt;                                // inclusive scan over the block
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == kWave - 1) s_wave[w] = x;
        __syncthreads();
        if (w == 0) {
            int v = lane < kPlanThreads / kWave ? s_wave[lane] : 0;
            for (int o = 1; o < kPlanThreads / kWave; o <<= 1) {
                const int y = __shfl_up(v, o);
                if (lane >= o) v += y;
            }
            if (lane < kPlanThreads / kWave) s_wave[lane] = v;
        }
        __syncthreads();
        s_off[t] = x - cnt + (w > 0 ? s_wave[w - 1] : 0);
        s_row0[t] = row0;
        s_p[t] = p;
        const int total = s_wave[kPlanThreads / kWave - 1];
        __syncthreads();
        const int nb = c.batch - b0 < kPlanThreads ? c.batch - b0 : kPlanThreads;
        for (int k = t; k < total; k += kPlanThreads) {
            int lo = 0, hi = nb - 1;                // the last sequence whose offset is <= k
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= k) lo = mid; else hi = mid - 1;
            }
            const int ps = s_p[lo];
            const int q = ((ps & 1) ? 0 : 1) + 2 * (k - s_off[lo]);   // rows at odd positions complete
            const int r = s_row0[lo] + q;
            plan[carry + k] = make_int4(r, b0 + lo, q > 0 ? r - 1 : -1, (ps + q) >> 1);
        }
        carry += total;
        __syncthreads();                            // before the next round reuses the arrays
    }
    if (t == 0) *count = carry;
}

// Block i runs on XCD i % 8 (round-robin dispatch); that XCD's j-th block
// takes row tile (i % 8) + 8 (j / 18) and channel tile j % 18, so an XCD
// sweeps all channels of one row tile before the next and its L2 holds the
// tile's token rows while every XCD reads the whole weight matrix once.
// Lane (ty, tx) of wave w owns entries 8 ty .. 8 ty + 7 and channels
// 4 tx .. 4 tx + 3 of the tile for run w.  Per term block each wave stages
// u's 18 terms of its 64 entries ([term][entry]) and W's of its 32 channels
// ([term][channel]) in its own LDS area, prefetching the next block into
// registers while it computes.
__global__ __launch_bounds__(kTcThreads) void compress_tiled_kernel(AppendArgs a, const int4 *plan,
                                                                    const int32_t *count)
{
    __shared__ __attribute__((aligned(16))) float lds[kTcLdsFloats];
    __shared__ int s_rows[kTcRows];
    const int n = *count;
    const int i = blockIdx.x, j = i >> 3;
    const int rt = (i & 7) + 8 * (j / kTcChTiles), ct = j % kTcChTiles;
    const int k0 = rt * kTcRows;
    if (k0 >= n) return;
    const int c0 = ct * kTcCh;
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int ty = lane >> 3, tx = lane & 7;
    float *U = lds + w * kTcOpFloats;               // [18][64]
    float *Wt = U + kCompTerms * kTcRows;           // [18][32]
    float *R = lds + kTcRuns * kTcOpFloats;         // run sums [8][64][32]

    // staging sources of this lane: entry `lane` of the tile (run w's terms
    // lie in x_even for w < 4, in x_odd after), and W row c0 + (lane & 31),
    // half (lane >> 5) of each block's 18 terms.  Entries past the list
    // read token row 0 and are never stored.
    const int k = k0 + lane;
    const float *usrc = a.tokens;
    if (k < n) {
        const int4 pl = plan[k];
        usrc = w < kTcRuns / 2 ? (pl.z >= 0 ? a.tokens + (size_t)pl.z * kDim : a.c.pending + (size_t)pl.y * kDim)
                               : a.tokens + (size_t)pl.x * kDim;
        if (w == 0) s_rows[lane] = pl.x;
    }
    usrc += (w % (kTcRuns / 2)) * kTcRunBlocks * kCompTerms;
    const float *wsrc = a.w_comp + (size_t)(c0 + (lane & 31)) * (2 * kDim) + w * kTcRunBlocks * kCompTerms
                      + (lane >> 5) * (kCompTerms / 2);

    float2 pu[kCompTerms / 2];
    float pw[kCompTerms / 2];
    auto fetch = [&](int lb) {
        const float2 *u2 = reinterpret_cast<const float2 *>(usrc + lb * kCompTerms);
#pragma unroll
        for (int t = 0; t < kCompTerms / 2; ++t) pu[t] = u2[t];
        const float *wp = wsrc + lb * kCompTerms;
#pragma unroll
        for (int t = 0; t < kCompTerms / 2; ++t) pw[t] = wp[t];
    };

    // one term block of the run: stage the prefetched operands, prefetch the
    // next block, fold the 18 terms from +0 into acc
    // The operand area is the wave's own and one wave's LDS operations run
    // in issue order, so the wave only fences its own accesses (the
    // compiler may not move LDS reads across the writes), with no block
    // barrier.
    auto block = [&](int lb, float (&acc)[8][4]) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < kCompTerms / 2; ++t) {
            U[(2 * t) * kTcRows + lane] = pu[t].x;
            U[(2 * t + 1) * kTcRows + lane] = pu[t].y;
            Wt[((lane >> 5) * (kCompTerms / 2) + t) * kTcCh + (lane & 31)] = pw[t];
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (lb + 1 < kTcRunBlocks) fetch(lb + 1);
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[r][q] = 0.0f;
#pragma unroll 2
        for (int t = 0; t < kCompTerms; ++t) {
            const float4 ua = *reinterpret_cast<const float4 *>(U + t * kTcRows + 8 * ty);
            const float4 ub = *reinterpret_cast<const float4 *>(U + t * kTcRows + 8 * ty + 4);
            const float4 wv = *reinterpret_cast<const float4 *>(Wt + t * kTcCh + 4 * tx);
            const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
            const float ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(ww[q], uu[r], acc[r][q]);
        }
    };
    // x += y over the thread's outputs (fp32 addition is commutative, so the
    // operand order within one addition does not matter)
    auto add = [](float (&x)[8][4], const float (&y)[8][4]) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) x[r][q] = x[r][q] + y[r][q];
    };

    // the run's pairwise tree, written out.  The first half's sum waits in
    // this lane's own slots of the run-sum area (same lane, same addresses:
    // no barrier) so that three arrays are live at a time, not four.
    float *mine = R + (w * kTcRows + 8 * ty) * kTcCh + 4 * tx;
    float lv0[8][4], lv1[8][4], acc[8][4];
    fetch(0);
    block(0, lv0);
    block(1, acc);
    add(lv0, acc);                                  // b0 + b1
    block(2, lv1);
    block(3, acc);
    add(lv1, acc);                                  // b2 + b3
    add(lv0, lv1);                                  // (b0 + b1) + (b2 + b3)
#pragma unroll
    for (int r = 0; r < 8; ++r)
        *reinterpret_cast<float4 *>(mine + r * kTcCh) = make_float4(lv0[r][0], lv0[r][1], lv0[r][2], lv0[r][3]);
    block(4, lv0);
    block(5, acc);
    add(lv0, acc);                                  // b4 + b5
    block(6, lv1);
    block(7, acc);
    add(lv1, acc);                                  // b6 + b7
    add(lv0, lv1);                                  // (b4 + b5) + (b6 + b7)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float4 *m = reinterpret_cast<float4 *>(mine + r * kTcCh);
        const float4 h = *m;
        *m = make_float4(h.x + lv0[r][0], h.y + lv0[r][1], h.z + lv0[r][2], h.w + lv0[r][3]);
    }
    __syncthreads();
    for (int o = threadIdx.x; o < kTcRows * kTcCh; o += kTcThreads) {
        const int row = o / kTcCh, ch = o % kTcCh;
        if (k0 + row >= n) break;                   // o grows with row
        float P[kTcRuns];
#pragma unroll
        for (int p = 0; p < kTcRuns; ++p) P[p] = R[(p * kTcRows + row) * kTcCh + ch];
        const float e = ((P[0] + P[1]) + (P[2] + P[3])) + ((P[4] + P[5]) + (P[6] + P[7]));
        a.ent[(size_t)s_rows[row] * kDim + c0 + ch] = e;
    }
}

// ------------------------------------------------- matrix-core compressor
//
// The same listed entries as a product on the matrix cores, for callers
// that take a stated error instead of the fixed fp32 order [P1 §3.2: the
// compressor is a learned projection; a chunk of them is one product
// E = U W^T, U = the listed entries' x_even || x_odd rows].  Every fp32
// operand is split into bf16 high and low parts (x = hi + lo + d,
// |d| <= 2^-16 |x|) and each term is taken as hi*hi + hi*lo + lo*hi with
// v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation).  Per
// output the dropped parts are at most 3.02 * 2^-16 sum_j |W_rj u_j| and an
// fp32 sum of 3456 terms in any order adds at most 3455 * 2^-24 of the sum
// of their magnitudes, so |e - sum_j W_rj u_j| <= 2.53e-4 sum_j |W_rj u_j|.
//
// W is split once per call into the workspace, in the MFMA's B-operand
// order: for channel tile ct (16 channels) and contraction step s (32
// terms), 64 lanes x 8 bf16, lane l holding channel 16 ct + l % 16, terms
// 32 s + 8 (l / 16) .. + 7; the high part's 1 KB, then the low part's.
//
// A block takes 128 listed entries x 128 output channels (the last column
// of blocks covers channels 512 .. 575 and computes 64 more that it does not
// store); its four waves, 2 x 2, take 64 entries x 64 channels each, 4 x 4
// MFMA tiles.  Per contraction step the block stages in LDS, double-
// buffered: A, its entries' 32 terms split into bf16 high and low parts in
// the MFMA A-operand order (per 16-entry tile the high part's 64 lanes x
// 16 B, then the low part's: 16 KB), and B, the 8 channel tiles' pre-split
// W operands (16 KB) as the workspace holds them.  A wave reads its step's
// 4 A and 4 B operand pairs into registers, issues the loads of the next
// step's W and of the terms two steps ahead, runs its 48 MFMAs, writes the
// next step's W and split terms into the other buffer and meets the block
// at a barrier.  Each A and B operand thus serves 4 tiles (the former layout, a
// wave of 16 entries x 64 channels reading its W operands from L2 every
// step, was bound by that traffic).
constexpr int kMcRows = 128;                       // listed entries per block
constexpr int kMcCh = 128;                         // output channels per block
constexpr int kMcThreads = 256;
constexpr int kMcSteps = 2 * kDim / 32;            // 36 contraction steps of 32 terms
constexpr int kMcChTiles = kDim / 16;              // 36 channel tiles of 16
constexpr int kMcColBlocks = (kDim + kMcCh - 1) / kMcCh;   // 5
constexpr int kMcHalf = 16384;                     // A (or B) bytes of one stage
constexpr size_t kWsplitBytes = (size_t)kMcChTiles * kMcSteps * 2 * 1024;   // 2.65 MB

typedef __bf16 mc_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float mc_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((mc_f32x2_t{a, b}), mc_bf16x2_t));
}

// hi/lo bf16 split of 8 floats (round to nearest even both times)
__device__ __forceinline__ void split_bf16x8(const float4 &x0, const float4 &x1, u32x4_t &hi, u32x4_t &lo)
{
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = cvt_bf16x2(xv[2 * i], xv[2 * i + 1]);
        hi[i] = h;
        lo[i] = cvt_bf16x2(xv[2 * i] - __uint_as_float(h << 16), xv[2 * i + 1] - __uint_as_float(h & 0xFFFF0000u));
    }
}

// One thread per (channel tile, step, lane): 8 terms of one W row split.
__global__ __launch_bounds__(256) void split_w_kernel(const float *w_comp, uint8_t *wsplit)
{
    const int g = blockIdx.x * 256 + threadIdx.x;
    if (g >= kMcChTiles * kMcSteps * kWave) return;
    const int lane = g & (kWave - 1), step = (g / kWave) % kMcSteps, ct = g / (kWave * kMcSteps);
    const float *src = w_comp + (size_t)(16 * ct + (lane & 15)) * (2 * kDim) + 32 * step + 8 * (lane >> 4);
    u32x4_t hi, lo;
    split_bf16x8(*reinterpret_cast<const float4 *>(src), *reinterpret_cast<const float4 *>(src + 4), hi, lo);
    uint8_t *dst = wsplit + ((size_t)ct * kMcSteps + step) * 2048 + 16 * lane;
    *reinterpret_cast<u32x4_t *>(dst) = hi;
    *reinterpret_cast<u32x4_t *>(dst + 1024) = lo;
}

__global__ __launch_bounds__(kMcThreads, 2) void compress_mfma_kernel(AppendArgs a, const int4 *plan,
                                                                      const int32_t *count, const uint8_t *wsplit)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kMcHalf];     // 2 stages x (A, B)
    const int n = *count;
    const int k0 = blockIdx.x * kMcRows;
    if (k0 >= n) return;
    const int ct0 = blockIdx.y * (kMcCh / 16);
    const int t = threadIdx.x, w = t / kWave, lane = t & (kWave - 1);
    const int wr = w >> 1, wc = w & 1;             // the wave's 64 entries and 64 channels
    const int r16 = lane & 15, oct = lane >> 4;

    // U loads: thread t takes entry lr of the block (terms 16 lh .. 16 lh +
    // 15 of each step: two octets, all of x_even or all of x_odd)
    const int lr = t >> 1, lh = t & 1;
    const int rec = k0 + lr;
    const int4 pl = rec < n ? plan[rec] : make_int4(-1, 0, -1, 0);
    const float *xe = pl.x < 0 ? a.tokens
                    : pl.z >= 0 ? a.tokens + (size_t)pl.z * kDim : a.c.pending + (size_t)pl.y * kDim;
    const float *xo = pl.x < 0 ? a.tokens : a.tokens + (size_t)pl.x * kDim;
    // the terms of a step are loaded two steps ahead, into two register sets
    // used in turn
    float4 ua[4], ub[4];
    auto load_u = [&](int s, float4 (&d)[4]) {
        const int kk = 32 * s + 16 * lh;
        const float *src = kk < kDim ? xe + kk : xo + (kk - kDim);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = *reinterpret_cast<const float4 *>(src + 4 * i);
    };
    auto store_u = [&](uint8_t *A, const float4 (&u)[4]) {
        uint8_t *tile = A + (lr >> 4) * 2048;
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            u32x4_t hi, lo;
            split_bf16x8(u[2 * o], u[2 * o + 1], hi, lo);
            const int ln = (lr & 15) + 16 * (2 * lh + o);
            *reinterpret_cast<u32x4_t *>(tile + 16 * ln) = hi;
            *reinterpret_cast<u32x4_t *>(tile + 1024 + 16 * ln) = lo;
        }
    };
    // W: 16 pieces of 1 KB (channel tile q / 2, its high or low part), wave
    // w loading pieces 4w .. 4w + 3 into registers a step ahead; tiles past
    // the channels re-read the last one (their results are not stored).
    // (Through registers rather than LDS DMA: a block barrier's fence waits
    // for outstanding LDS DMA, and with it for the term loads behind it.)
    u32x4_t wv[4];
    auto load_w = [&](int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 4 * w + i;
            const int ct = ct0 + (q >> 1) < kMcChTiles ? ct0 + (q >> 1) : kMcChTiles - 1;
            wv[i] = *reinterpret_cast<const u32x4_t *>(wsplit + ((size_t)ct * kMcSteps + s) * 2048 +
                                                       1024 * (q & 1) + 16 * lane);
        }
    };
    auto store_w = [&](uint8_t *B) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t *>(B + 1024 * (4 * w + i) + 16 * lane) = wv[i];
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step s: products from stage s % 2; meanwhile W of step s + 1 is loaded
    // and the terms of step s + 2 into `ld`; at the end W and the terms of
    // step s + 1 (in `st`, loaded a step ago) go into the other stage.
    auto step = [&](int s, const float4 (&st)[4], float4 (&ld)[4]) {
        const uint8_t *cur = lds + (s & 1) * 2 * kMcHalf;
        uint8_t *nxt = lds + ((s + 1) & 1) * 2 * kMcHalf;
        u32x4_t ah[4], al[4], bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t *pa = cur + (4 * wr + i) * 2048 + 16 * lane;
            ah[i] = *reinterpret_cast<const u32x4_t *>(pa);
            al[i] = *reinterpret_cast<const u32x4_t *>(pa + 1024);
            const uint8_t *pb = cur + kMcHalf + (4 * wc + i) * 2048 + 16 * lane;
            bh[i] = *reinterpret_cast<const u32x4_t *>(pb);
            bl[i] = *reinterpret_cast<const u32x4_t *>(pb + 1024);
        }
        const bool more = s + 1 < kMcSteps, more2 = s + 2 < kMcSteps;
        if (more) load_w(s + 1);
        if (more2) load_u(s + 2, ld);
        __builtin_amdgcn_sched_barrier(0);          // the loads go out before the products
        // high x high for all 16 tiles, then high x low, then low x high, so
        // that consecutive products of one accumulator are 16 apart
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(ah[i], bh[j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(ah[i], bl[j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(al[i], bh[j], acc[i][j]);
        if (more) {
            store_u(nxt, st);
            store_w(nxt + kMcHalf);
        }
        __syncthreads();
    };

    load_w(0);
    load_u(0, ub);
    load_u(1, ua);
    store_w(lds + kMcHalf);
    store_u(lds, ub);
    __syncthreads();
    static_assert(kMcSteps % 2 == 0, "steps go in pairs");
    for (int s = 0; s < kMcSteps; s += 2) {
        step(s, ua, ub);                           // stores step s + 1 from ua, loads step s + 2 into ub
        step(s + 1, ub, ua);
    }
    // D layout: lane holds entries 4 oct .. 4 oct + 3 of column r16 of each tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rr = k0 + 64 * wr + 16 * i + 4 * oct + v;
            if (rr >= n) continue;
            float *erow = a.ent + (size_t)plan[rr].x * kDim;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ch = 16 * (ct0 + 4 * wc + j) + r16;
                if (ch < kDim) erow[ch] = acc[i][j][v];
            }
        }
}

// Quantiser of a planned append: kQPer listed entries per block, the
// compressor's output read from the entry's input row.
constexpr int kQPer = 4;
__global__ __launch_bounds__(kAppendThreads) void quantize_planned_kernel(AppendArgs a, const int4 *plan,
                                                                          const int32_t *count)
{
    __shared__ float wave_max[kAppendThreads / kWave];
    const int n = *count;
    const int k0 = blockIdx.x * kQPer;
    if (k0 >= n) return;
    const int t = threadIdx.x;
    int4 pl[kQPer];
    float e[kQPer];
    uint16_t key[kQPer];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) pl[i] = k0 + i < n ? plan[k0 + i] : make_int4(-1, 0, -1, 0);
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
        const int64_t row = pl[i].x >= 0 ? pl[i].x : 0;
        e[i] = a.ent[(size_t)row * kDim + t];
        key[i] = a.idx_rows[(size_t)row * a.c.idx_dim + (t < a.c.idx_dim ? t : 0)];
    }
#pragma unroll
    for (int i = 0; i < kQPer; ++i)
        if (pl[i].x >= 0) {                         // uniform over the block
            const int64_t slot = plane_row(a.c, pl[i].y, pl[i].w);
            if (slot >= 0) quantize_entry(a, e[i], t, (size_t)slot, key[i], wave_max);
            else if (t == 0) atomicOr(a.c.status, CSKV_STATUS_BAD_PAGE);
        }
}

// Quantiser of a planned append for caches with fp32 group scales and bf16
// indexer keys: one wave per listed entry, no block barrier.  Lane l holds
// the latent channels 8 l .. 8 l + 7 (it packs their codes into one word
// itself) and RoPE channel 512 + l.  A group of g latent channels spans g/8
// lanes; the RoPE channels (g = 32 or 64 inside 64 lanes) reduce and pack
// with lane exchanges.  Same arithmetic as quantize_channel: absmax, s =
// absmax / 6 by IEEE division, codes of x / s.
constexpr int kQwWaves = 4;
__device__ __forceinline__ float xor_max(float a, int lanes)
{
    for (int off = 1; off < lanes; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
    return a;
}

// The code word of one lane's 8 latent channels with group g (g >= 8) into
// plane row `codes` / `scales`.
__device__ __forceinline__ void quantize_lane8(const float (&x)[8], int lane, int g, uint8_t *codes, float *scales)
{
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
    a = xor_max(a, g / 8);
    const float s = a / 6.0f;                      // IEEE division (no fast-math)
    uint32_t word = 0;
    if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(x[i] / s) << (4 * i);
    }
    reinterpret_cast<uint32_t *>(codes)[lane] = word;
    if ((lane % (g / 8)) == 0) scales[lane / (g / 8)] = s;
}

__global__ __launch_bounds__(kQwWaves * kWave) void quantize_planned_wave_kernel(AppendArgs a, const int4 *plan,
                                                                                 const int32_t *count)
{
    const cskv_cache &c = a.c;
    const int n = *count;
    const int k = blockIdx.x * kQwWaves + threadIdx.x / kWave;
    if (k >= n) return;                             // whole waves
    const int lane = threadIdx.x & (kWave - 1);
    const int4 pl = plan[k];
    const float *row = a.ent + (size_t)pl.x * kDim;
    const float4 lo = reinterpret_cast<const float4 *>(row)[2 * lane];
    const float4 hi = reinterpret_cast<const float4 *>(row)[2 * lane + 1];
    const float xr = row[8 * kWave + lane];
    const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const int64_t prow = plane_row(c, pl.y, pl.w);
    if (prow < 0) {                                 // whole waves
        if (lane == 0) atomicOr(c.status, CSKV_STATUS_BAD_PAGE);
        return;
    }
    const size_t slot = (size_t)prow;
    const int kg = c.k_group;
    uint8_t *kc = c.k_codes + slot * (kDim / 2);
    float *ks = c.k_scales + slot * (kDim / kg);
    quantize_lane8(x, lane, kg, kc, ks);
    {   // RoPE channels 512 .. 575: groups of kg lanes
        const float ar = xor_max(fabsf(xr), kg);
        const float sr = ar / 6.0f;
        uint32_t code = sr != 0.0f ? e2m1_code(xr / sr) : 0u;
        code |= __shfl_down(code, 1) << 4;
        code |= __shfl_down(code, 2) << 8;
        code |= __shfl_down(code, 4) << 16;
        if ((lane & 7) == 0) *reinterpret_cast<uint32_t *>(kc + 4 * kWave + lane / 2) = code;
        if ((lane % kg) == 0) ks[(8 * kWave + lane) / kg] = sr;
    }
    if (c.v_group > 0) {
        const int dv = c.dim - c.rope_dim;          // 512: the latent channels
        quantize_lane8(x, lane, c.v_group, c.v_codes + slot * (dv / 2), c.v_scales + slot * (dv / c.v_group));
    }
    if (c.idx_dim == 2 * kWave)
        reinterpret_cast<uint32_t *>(c.idx_keys + slot * c.idx_dim)[lane] =
            reinterpret_cast<const uint32_t *>(a.idx_rows + (size_t)pl.x * c.idx_dim)[lane];
    else
        c.idx_keys[slot * c.idx_dim + lane] = a.idx_rows[(size_t)pl.x * c.idx_dim + lane];
}

// Workspace of an append with the compressor: the compressor's fp32 rows,
// then the plan records and their count.
struct AppendWs {
    size_t plan_off, count_off, wsplit_off, total;
};
inline AppendWs append_ws_layout(int64_t total_new)
{
    AppendWs L;
    L.plan_off = ((size_t)total_new * kDim * sizeof(float) + 255) / 256 * 256;
    L.count_off = L.plan_off + ((size_t)total_new * sizeof(int4) + 255) / 256 * 256;
    L.wsplit_off = L.count_off + 256;
    L.total = L.wsplit_off + (total_new >= kTiledMinRows ? kWsplitBytes : 0);
    return L;
}

}  // namespace

size_t append_workspace_bytes(int total_new)
{
    return append_ws_layout(total_new).total;
}

hipError_t launch_kv_append(const cskv_cache &c, const float *tokens, const int32_t *cu_new,
                            int total_new, const float *w_comp, const uint16_t *idx_rows,
                            void *ws, hipStream_t s, uint16_t *swa_ring, const float *swa_rows,
                            int swa_window, bool mfma)
{
    if (total_new == 0) return hipSuccess;
    AppendArgs a{c, tokens, cu_new, w_comp, idx_rows, static_cast<float *>(ws), total_new,
                 cu_new ? nullptr : swa_ring, swa_rows, swa_window};
    TimedLaunch tl = timer_take(CSKV_KERNEL_APPEND);
    // one row per sequence: the quantiser also finalises (one launch less)
    const bool fused = cu_new == nullptr;
    const dim3 qgrid((unsigned)total_new), qblock(kAppendThreads);
    if (w_comp && cu_new && total_new >= kTiledMinRows) {
        // a large append: plan, tiled compressor, planned quantiser, finalise
        const TimedLaunch tc = timer_take(CSKV_KERNEL_COMPRESS);
        hipEvent_t comp_start = tl.start;
        if (tc.start) comp_start = tc.start;
        else tl.start = nullptr;
        const AppendWs L = append_ws_layout(total_new);
        int4 *plan = reinterpret_cast<int4 *>(static_cast<char *>(ws) + L.plan_off);
        int32_t *count = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + L.count_off);
        const int64_t bound = plan_bound(total_new, c.batch);
        const int64_t row_tiles8 = ((bound + kTcRows - 1) / kTcRows + 7) / 8 * 8;
        launch_kernel(compress_plan_kernel, dim3(1), dim3(kPlanThreads), s, comp_start, nullptr, a, plan, count);
        if (mfma) {
            uint8_t *wsplit = static_cast<uint8_t *>(ws) + L.wsplit_off;
            launch_kernel(split_w_kernel, dim3((unsigned)((kMcChTiles * kMcSteps * kWave + 255) / 256)), dim3(256),
                          s, nullptr, nullptr, w_comp, wsplit);
            launch_kernel(compress_mfma_kernel, dim3((unsigned)((bound + kMcRows - 1) / kMcRows), kMcColBlocks),
                          dim3(kMcThreads), s, nullptr, tc.stop, a, (const int4 *)plan, (const int32_t *)count,
                          (const uint8_t *)wsplit);
        }
        else
            launch_kernel(compress_tiled_kernel, dim3((unsigned)(row_tiles8 * kTcChTiles)), dim3(kTcThreads), s,
                          nullptr, tc.stop, a, (const int4 *)plan, (const int32_t *)count);
        if (c.k_format == CSKV_KV_F32 && c.idx_format == CSKV_IDX_BF16)
            launch_kernel(quantize_planned_wave_kernel, dim3((unsigned)((bound + kQwWaves - 1) / kQwWaves)),
                          dim3(kQwWaves * kWave), s, tl.start, nullptr, a, (const int4 *)plan,
                          (const int32_t *)count);
        else
            launch_kernel(quantize_planned_kernel, dim3((unsigned)((bound + kQPer - 1) / kQPer)), qblock, s,
                          tl.start, nullptr, a, (const int4 *)plan, (const int32_t *)count);
        launch_kernel(append_finalize_kernel<true>, dim3((unsigned)c.batch), dim3(kWave), s, nullptr, tl.stop, a);
    } else if (w_comp) {
        // the compressor timed alone: the append interval starts after it
        const TimedLaunch tc = timer_take(CSKV_KERNEL_COMPRESS);
        hipEvent_t comp_start = tl.start;
        if (tc.start) comp_start = tc.start;
        else tl.start = nullptr;
        // about 1024 waves: groups of E input rows x runs of output channels;
        // E = 4 for a few rows (a 32-sequence decode step: 12.4 -> 11.2 us
        // against E = 8), 8 beyond (255 rows: 24 us against 28 with E = 4)
        auto compress = [&](auto e) {
            constexpr int kE = decltype(e)::value;
            const int groups = (total_new + kE - 1) / kE;
            const int runs = groups >= 1024 ? 1 : (1024 / groups < kDim ? 1024 / groups : kDim);
            const int cpw = (kDim + runs - 1) / runs;
            launch_kernel(compress_kernel<kE>, dim3((unsigned)((kDim + cpw - 1) / cpw), (unsigned)groups),
                          dim3(kWave), s, comp_start, tc.stop, a, cpw);
        };
        if (total_new <= 64) compress(std::integral_constant<int, 4>{});
        else compress(std::integral_constant<int, 8>{});
        if (fused) {
            launch_kernel(quantize_kernel<true, true>, qgrid, qblock, s, tl.start, tl.stop, a);
        } else {
            launch_kernel(quantize_kernel<true, false>, qgrid, qblock, s, tl.start, nullptr, a);
            launch_kernel(append_finalize_kernel<true>, dim3((unsigned)c.batch), dim3(kWave), s, nullptr, tl.stop, a);
        }
    } else if (fused) {
        launch_kernel(quantize_kernel<false, true>, qgrid, qblock, s, tl.start, tl.stop, a);
    } else {
        launch_kernel(quantize_kernel<false, false>, qgrid, qblock, s, tl.start, nullptr, a);
        launch_kernel(append_finalize_kernel<false>, dim3((unsigned)c.batch), dim3(kWave), s, nullptr, tl.stop, a);
    }
    return hipGetLastError();
}

static size_t deferred_ent_bytes(int batch) { return ((size_t)batch * kDim * sizeof(float) + 255) / 256 * 256; }

size_t deferred_entry_bytes(int batch)
{
    return deferred_ent_bytes(batch) + ((size_t)batch * sizeof(int64_t) + 255) / 256 * 256;
}

DeferredEntry deferred_entry_at(void *base, int batch, const float *tokens, const float *w_comp)
{
    char *p = static_cast<char *>(base);
    return DeferredEntry{tokens, w_comp, reinterpret_cast<float *>(p),
                         reinterpret_cast<int64_t *>(p + deferred_ent_bytes(batch))};
}

hipError_t launch_append_head(const cskv_cache &c, const DeferredEntry &d, const uint16_t *idx_rows,
                              hipStream_t s, uint16_t *swa_ring, const float *swa_rows, int swa_window)
{
    const AppendArgs a{c, d.tokens, nullptr, d.w_comp, idx_rows, d.ent, c.batch, swa_ring, swa_rows, swa_window,
                       d.slots};
    const TimedLaunch tl = timer_take(CSKV_KERNEL_APPEND);
    launch_kernel(quantize_kernel<true, true, true>, dim3((unsigned)c.batch), dim3(kAppendThreads), s, tl.start,
                  tl.stop, a);
    return hipGetLastError();
}

hipError_t launch_swa_append(uint16_t *ring, int batch, int window, int dim, const float *rows,
                             const int32_t *cu_new, int total_new, const int32_t *end_pos,
                             hipStream_t s, bool fp8)
{
    if (total_new == 0) return hipSuccess;
    SwaArgs a{ring, batch, window, dim, rows, cu_new, end_pos, total_new};
    const TimedLaunch tl = timer_take(CSKV_KERNEL_SWA_APPEND);
    if (fp8)
        launch_kernel(swa_append_kernel<true>, dim3((unsigned)total_new), dim3(kWave), s, tl.start, tl.stop, a);
    else
        launch_kernel(swa_append_kernel<false>, dim3((unsigned)total_new), dim3(kWave), s, tl.start, tl.stop, a);
    return hipGetLastError();
}

}  // namespace cskv
