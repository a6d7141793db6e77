// indexer.hip -- indexer scoring over every cached entry and exact top-k
// [P2 三、"突破四：滑动窗口和稀疏注意力" (a light indexer scores all history,
// attention keeps the 512 best); P2 四、"CSA2：三种模式" (per-layer multi-head
// indexer query, per-entry indexer key)].
//
// Scan: s_j = sum_h w_h * relu(q_h . K_j) is a [heads x dim] x [dim x entries]
// contraction, run on bf16 MFMA with fp32 accumulation.  Each block streams a
// contiguous run of one sequence's keys through LDS with coalesced 16-byte
// loads, scores them, writes an order-preserving uint32 key per entry and adds
// the entries to a per-sequence histogram of the keys' top 11 bits.
//
// Select: one block per sequence finds the k-th largest key by radix passes
// (11 + 11 + 10 bits; the first histogram comes from the scan), then writes the
// selected indices in ascending order, taking tied keys from the lowest index.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static size_t key_stride(const cskv_cache &c) { return align_up((size_t)c.capacity, 64); }

TopkWorkspace topk_workspace(const cskv_cache &c)
{
    TopkWorkspace w;
    w.keys_off = 0;
    w.hist_off = align_up(sizeof(uint32_t) * key_stride(c) * (size_t)c.batch, 256);
    w.total = align_up(w.hist_off + sizeof(uint32_t) * kHistBins * (size_t)c.batch, 256);
    return w;
}

namespace {

constexpr int kScanThreads = 256;   // 4 waves
constexpr int kTile = 64;           // entries per LDS tile: 16 per wave

struct ScanArgs {
    const uint16_t *keys;      // idx_keys plane
    const int32_t *n_tokens;
    const uint16_t *q;         // [B][H][Di]
    const float *head_w;       // [B][H] or null
    uint32_t *out_keys;        // [B][key_stride]
    uint32_t *hist;            // [B][kHistBins]
    int capacity, heads, chunk;
    size_t key_stride;
};

template <int DI>
__device__ __forceinline__ int swz(int row, int ch)
{
    // 16-byte chunk permutation inside a key row so that the 16 rows one MFMA
    // operand read touches fall on distinct LDS banks.
    return DI == 128 ? (ch ^ (row & 15)) : (ch ^ ((row >> 1) & 7));
}

template <int DI>
__global__ __launch_bounds__(kScanThreads) void indexer_scan_kernel(ScanArgs a)
{
    constexpr int kChunks = DI / 8;        // 16-byte chunks per key row
    constexpr int kSteps = DI / 32;        // MFMA contraction steps
    __shared__ u32x4_t tile[kTile * kChunks];
    __shared__ uint32_t hist[kHistBins];

    const int b = blockIdx.y;
    const int64_t E = entries_of(a.n_tokens, b, a.capacity);
    const int64_t e_begin = (int64_t)blockIdx.x * a.chunk;
    if (e_begin >= E) return;
    const int64_t e_end = E < e_begin + a.chunk ? E : e_begin + a.chunk;

    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    for (int i = t; i < kHistBins; i += kScanThreads) hist[i] = 0;

    // Indexer query as MFMA A operands: row = head (16 per tile), held for the
    // whole block.  Missing heads (H not a multiple of 16) are zero rows.
    const int mtiles = (a.heads + 15) / 16;
    u32x4_t qa[4][kSteps];
    float hw[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int head = 16 * mt + (lane & 15);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (mt < mtiles && head < a.heads)
                v = *reinterpret_cast<const u32x4_t *>(
                    a.q + ((size_t)b * a.heads + head) * DI + 32 * s + 8 * (lane >> 4));
            qa[mt][s] = v;
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int hrow = 16 * mt + 4 * (lane >> 4) + v;
            hw[mt][v] = hrow < a.heads ? (a.head_w ? a.head_w[(size_t)b * a.heads + hrow] : 1.0f) : 0.0f;
        }
    }

    const uint8_t *kb = reinterpret_cast<const uint8_t *>(a.keys + (size_t)b * a.capacity * DI);
    uint32_t *ok = a.out_keys + (size_t)b * a.key_stride;
    for (int64_t t0 = e_begin; t0 < e_end; t0 += kTile) {
        __syncthreads();   // previous tile fully consumed (and hist zeroed on entry)
        for (int ci = t; ci < kTile * kChunks; ci += kScanThreads) {
            const int row = ci / kChunks, ch = ci % kChunks;
            const int64_t e = t0 + row;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (e < e_end) v = *reinterpret_cast<const u32x4_t *>(kb + (size_t)e * (2 * DI) + 16 * ch);
            tile[row * kChunks + swz<DI>(row, ch)] = v;
        }
        __syncthreads();
        const int row = 16 * w + (lane & 15);
        f32x4_t acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const u32x4_t bop = tile[row * kChunks + swz<DI>(row, 4 * s + (lane >> 4))];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (mt < mtiles) acc[mt] = mfma16x16x32(qa[mt][s], bop, acc[mt]);
        }
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) part += hw[mt][v] * fmaxf(acc[mt][v], 0.f);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        const int64_t e = t0 + row;
        if (lane < 16 && e < e_end) {
            const uint32_t key = score_key(part);
            ok[e] = key;
            atomicAdd(&hist[key >> 21], 1u);
        }
    }
    __syncthreads();
    uint32_t *gh = a.hist + (size_t)b * kHistBins;
    for (int i = t; i < kHistBins; i += kScanThreads)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------- select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kCandMax = 6144;
constexpr int kPer = 4;                       // elements per thread per sweep
constexpr int kSweep = kSelThreads * kPer;

struct SelectArgs {
    const uint32_t *keys;
    const uint32_t *hist;
    const int32_t *n_tokens;
    int32_t *out;
    int capacity, k;
    size_t key_stride;
};

struct SelectSmem {
    uint32_t bins[kHistBins];
    uint32_t cand_key[kCandMax];
    int32_t cand_idx[kCandMax];
    uint32_t wave_sum[kSelWaves];
    uint32_t found[4];
};

// Inclusive prefix sum over the block; *total receives the block sum.
__device__ uint32_t block_scan(uint32_t v, uint32_t *wave_sum, uint32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t n = __shfl_up(v, off);
        if (lane >= off) v += n;
    }
    if (lane == kWave - 1) wave_sum[w] = v;
    __syncthreads();
    if (w == 0) {
        uint32_t x = lane < kSelWaves ? wave_sum[lane] : 0u;
        for (int off = 1; off < kSelWaves; off <<= 1) {
            const uint32_t n = __shfl_up(x, off);
            if (lane >= off) x += n;
        }
        if (lane < kSelWaves) wave_sum[lane] = x;
    }
    __syncthreads();
    const uint32_t base = w ? wave_sum[w - 1] : 0u;
    *total = wave_sum[kSelWaves - 1];
    __syncthreads();
    return v + base;
}

// Over a histogram of n bins held in sm.bins, find the highest bin t with
// (count of bins above t) < need <= (count of bins >= t).  Returns t and the
// count strictly above it.
__device__ void find_threshold_bin(SelectSmem &sm, int n, uint32_t need, uint32_t *bin,
                                   uint32_t *above)
{
    const int t = threadIdx.x;
    // thread t owns bins n-1-2t and n-2-2t (descending order)
    const int b0 = n - 1 - 2 * t, b1 = n - 2 - 2 * t;
    const uint32_t c0 = b0 >= 0 ? sm.bins[b0] : 0u, c1 = b1 >= 0 ? sm.bins[b1] : 0u;
    uint32_t total;
    const uint32_t incl = block_scan(c0 + c1, sm.wave_sum, &total);
    const uint32_t before = incl - c0 - c1;
    if (before < need && need <= before + c0) { sm.found[0] = (uint32_t)b0; sm.found[1] = before; }
    if (before + c0 < need && need <= incl && b1 >= 0) { sm.found[0] = (uint32_t)b1; sm.found[1] = before + c0; }
    __syncthreads();
    *bin = sm.found[0];
    *above = sm.found[1];
    __syncthreads();
}

// Elements come either from the candidate list in LDS or straight from the
// key array in global memory; both are visited in ascending index order.
struct FromLds {
    const SelectSmem *sm;
    int64_t n;
    __device__ uint32_t key(int64_t i) const { return sm->cand_key[i]; }
    __device__ int32_t index(int64_t i) const { return sm->cand_idx[i]; }
};
struct FromGlobal {
    const uint32_t *keys;
    int64_t n;
    __device__ uint32_t key(int64_t i) const { return keys[i]; }
    __device__ int32_t index(int64_t i) const { return (int32_t)i; }
};

// Histogram of `bits`-bit digit at `shift` over elements whose key >> (shift+bits)
// equals prefix.
template <class Src>
__device__ void digit_histogram(SelectSmem &sm, const Src &src, int shift, int bits, uint32_t prefix)
{
    const int nb = 1 << bits;
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) sm.bins[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < src.n; i += kSelThreads) {
        const uint32_t k = src.key(i);
        if ((k >> (shift + bits)) == prefix) atomicAdd(&sm.bins[(k >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
}

// Exact threshold T (the k-th largest key) and the number of keys above it,
// given the first-pass bin t1 and the count above that bin.
template <class Src>
__device__ void refine_threshold(SelectSmem &sm, const Src &src, uint32_t t1, uint32_t above1,
                                 uint32_t k, uint32_t *T, uint32_t *above)
{
    uint32_t t2, a2, t3, a3;
    digit_histogram(sm, src, 10, 11, t1);
    find_threshold_bin(sm, 2048, k - above1, &t2, &a2);
    const uint32_t p2 = (t1 << 11) | t2;
    digit_histogram(sm, src, 0, 10, p2);
    find_threshold_bin(sm, 1024, k - above1 - a2, &t3, &a3);
    *T = (p2 << 10) | t3;
    *above = above1 + a2 + a3;
}

// Write, in ascending index order, every element with key > T and the first
// `ties` elements with key == T.
template <class Src>
__device__ void emit_selected(SelectSmem &sm, const Src &src, uint32_t T, uint32_t ties,
                              int32_t *out, int k)
{
    uint32_t tie_base = 0, sel_base = 0;
    for (int64_t s0 = 0; s0 < src.n; s0 += kSweep) {
        uint32_t key[kPer];
        int32_t idx[kPer];
        uint32_t nt = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t e = s0 + (int64_t)threadIdx.x * kPer + i;
            const bool in = e < src.n;
            key[i] = in ? src.key(e) : 0u;
            idx[i] = in ? src.index(e) : -1;
            nt += (in && key[i] == T) ? 1u : 0u;
        }
        uint32_t tot_t;
        uint32_t tie_pos = tie_base + block_scan(nt, sm.wave_sum, &tot_t) - nt;
        bool sel[kPer];
        uint32_t ns = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool in = idx[i] >= 0;
            bool s = in && key[i] > T;
            if (in && key[i] == T) { s = tie_pos < ties; ++tie_pos; }
            sel[i] = s;
            ns += s ? 1u : 0u;
        }
        uint32_t tot_s;
        uint32_t pos = sel_base + block_scan(ns, sm.wave_sum, &tot_s) - ns;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (sel[i]) { if (pos < (uint32_t)k) out[pos] = idx[i]; ++pos; }
        tie_base += tot_t;
        sel_base += tot_s;
    }
    for (int i = (int)sel_base + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectArgs a)
{
    __shared__ SelectSmem sm;
    const int b = blockIdx.x, t = threadIdx.x;
    const int64_t E = entries_of(a.n_tokens, b, a.capacity);
    int32_t *out = a.out + (size_t)b * a.k;
    const uint32_t *keys = a.keys + (size_t)b * a.key_stride;
    if (E <= a.k) {
        for (int i = t; i < a.k; i += kSelThreads) out[i] = i < E ? i : -1;
        return;
    }
    // pass 1: top 11 bits, histogram built by the scan
    for (int i = t; i < kHistBins; i += kSelThreads) sm.bins[i] = a.hist[(size_t)b * kHistBins + i];
    __syncthreads();
    uint32_t t1, above1;
    find_threshold_bin(sm, kHistBins, (uint32_t)a.k, &t1, &above1);
    const uint32_t floor_key = t1 << 21;

    // ordered compaction of every key in bins >= t1 into the candidate list
    uint32_t base = 0;
    for (int64_t s0 = 0; s0 < E; s0 += kSweep) {
        uint32_t key[kPer];
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t e = s0 + (int64_t)t * kPer + i;
            key[i] = e < E ? keys[e] : 0u;
            n += (e < E && key[i] >= floor_key) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t pos = base + block_scan(n, sm.wave_sum, &tot) - n;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t e = s0 + (int64_t)t * kPer + i;
            if (e < E && key[i] >= floor_key) {
                if (pos < (uint32_t)kCandMax) { sm.cand_key[pos] = key[i]; sm.cand_idx[pos] = (int32_t)e; }
                ++pos;
            }
        }
        base += tot;
    }
    __syncthreads();

    uint32_t T, above;
    if (base <= (uint32_t)kCandMax) {
        FromLds src{&sm, (int64_t)base};
        refine_threshold(sm, src, t1, above1, (uint32_t)a.k, &T, &above);
        emit_selected(sm, src, T, (uint32_t)a.k - above, out, a.k);
    } else {
        FromGlobal src{keys, E};
        refine_threshold(sm, src, t1, above1, (uint32_t)a.k, &T, &above);
        emit_selected(sm, src, T, (uint32_t)a.k - above, out, a.k);
    }
}

}  // namespace

hipError_t launch_indexer_topk(const cskv_cache &c, const uint16_t *q_idx, int heads,
                               const float *head_w, int k, int32_t *out_idx, void *ws,
                               hipStream_t s)
{
    const TopkWorkspace lay = topk_workspace(c);
    uint32_t *keys = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.keys_off);
    uint32_t *hist = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.hist_off);
    const size_t nh = (size_t)kHistBins * c.batch;
    zero_u32_kernel<<<(unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024), 256, 0, s>>>(hist, nh);

    // entries per block: aim for ~2048 blocks over the batch, 256..4096, a
    // multiple of the tile
    size_t chunk = ((size_t)c.capacity * c.batch + 2047) / 2048;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    chunk = chunk < 256 ? 256 : (chunk > 4096 ? 4096 : chunk);
    ScanArgs sa{c.idx_keys, c.n_tokens, q_idx, head_w, keys, hist, c.capacity, heads, (int)chunk,
                key_stride(c)};
    dim3 grid((unsigned)(((size_t)c.capacity + chunk - 1) / chunk), (unsigned)c.batch);
    timer_before(CSKV_KERNEL_INDEXER_SCAN, s);
    if (c.idx_dim == 128)
        indexer_scan_kernel<128><<<grid, kScanThreads, 0, s>>>(sa);
    else
        indexer_scan_kernel<64><<<grid, kScanThreads, 0, s>>>(sa);
    timer_after(CSKV_KERNEL_INDEXER_SCAN, s);

    SelectArgs se{keys, hist, c.n_tokens, out_idx, c.capacity, k, key_stride(c)};
    timer_before(CSKV_KERNEL_TOPK_SELECT, s);
    topk_select_kernel<<<c.batch, kSelThreads, 0, s>>>(se);
    timer_after(CSKV_KERNEL_TOPK_SELECT, s);
    return hipGetLastError();
}

}  // namespace cskv
