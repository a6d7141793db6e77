// indexer.hip -- indexer top-k: the scan (scan.hip) scores every cached
// entry, then the k best are selected [P2 三、"突破四：滑动窗口和稀疏注意力"
// (a light indexer scores all history, attention keeps the 512 best); P2 四、
// "CSA2：三种模式" (per-layer multi-head indexer query, per-entry indexer key)].
//
// Select: exact top-k per sequence by radix select on those keys.  The digit
// windows adapt to the keys' actual range (the first window starts below the
// common prefix of the smallest and largest key).  Caches of up to 128K
// entries per sequence take the tile select: the scan also writes the
// largest key of every 16-entry tile, and the k-th largest of those tile
// maxima is a lower bound of the k-th largest key (k tiles each hold a key at
// least that large).  One block per sequence finds that bound by radix select
// over the tile maxima, keeps the keys at or above it (a few more than k for
// scores without heavy ties) in index order, and selects the top k among
// them.  Longer caches are cut into slices of 4096 keys, one block each,
// whose local top-k lists (which must contain the global top-k) are merged by
// one block per sequence; a sequence of at most one slice is selected
// directly.  The output lists the selected indices in ascending order; among
// equal scores the lower index wins.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include <type_traits>

#include "append_dev.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Keys per slice: caches of few sequences (whose slices alone leave most of
// the chip idle) longer than one 4096-key slice take slices of 8192 keys on
// 1024-thread blocks, which halves the lists to merge; others slices of 4096
// keys on 512 threads.  (One 1M-token sequence: 85 -> 73 us per decode step;
// at 32 sequences the larger slices were slower.)
constexpr int kFewSeqs = 4;
static int slice_keys_of(const cskv_cache &c)
{
    return c.batch <= kFewSeqs && c.capacity > kSliceKeys ? 2 * kSliceKeys : kSliceKeys;
}
int topk_slices(const cskv_cache &c)
{
    const int sk = slice_keys_of(c);
    return (int)((c.capacity + sk - 1) / sk);
}

// Candidate pairs per sequence, rounded to even so each list is 16-byte aligned.
static size_t cand_stride(const cskv_cache &c, int k) { return ((size_t)topk_slices(c) * k + 1) & ~(size_t)1; }

// Caches of many slices merge in two levels: blocks of kGroupSlices slice
// lists first (one block each, in parallel), then the groups' lists.  One
// merge block over 122 lists of 512 (a 1M-token sequence) ran 4 rounds of
// its select; two levels keep every select to one round.
constexpr int kGroupSlices = 8;
constexpr int kGroupMinSlices = 25;
static int topk_groups(const cskv_cache &c, int k)
{
    const int s = topk_slices(c);
    return s >= kGroupMinSlices && k < slice_keys_of(c) ? (s + kGroupSlices - 1) / kGroupSlices : 0;
}
static size_t cand2_stride(const cskv_cache &c, int k) { return ((size_t)topk_groups(c, k) * k + 1) & ~(size_t)1; }

// The bound select serves caches longer than one slice and at most
// kTileMaxCap entries per sequence.  Its bound comes from at most 8192
// maxima per sequence: the 16-entry tiles' up to 131,072 entries, beyond
// that the maxima of groups of 2 or 4 consecutive tiles (tile_group).
constexpr int kTileMaxCap = 1 << 19;
static bool topk_uses_tiles(const cskv_cache &c)
{
    return c.capacity > kSliceKeys && c.capacity <= kTileMaxCap;
}
static int tile_group(const cskv_cache &c) { return c.capacity <= (1 << 17) ? 1 : c.capacity <= (1 << 18) ? 2 : 4; }
static size_t tile_stride(const cskv_cache &c) { return ((size_t)c.capacity / 16 + 1 + 63) / 64 * 64; }
static int bound_slices(const cskv_cache &c) { return (int)((c.capacity + kSliceKeys - 1) / kSliceKeys); }

TopkWorkspace topk_workspace(const cskv_cache &c, int k)
{
    TopkWorkspace w;
    w.keys_off = 0;
    w.cand_off = align_up(sizeof(uint32_t) * score_key_stride(c) * (size_t)c.batch, 256);
    if (topk_uses_tiles(c)) {
        // per sequence: one candidate list of up to kSliceKeys pairs per slice,
        // the slices' counts, the tile maxima
        w.tiles = true;
        w.cand2_off = w.cand_off;
        const size_t slices = (size_t)bound_slices(c);
        w.tcand_off = w.cand_off;
        const size_t tcount_off = align_up(w.tcand_off + sizeof(uint2) * slices * kSliceKeys * c.batch, 256);
        w.tmax_off = align_up(tcount_off + sizeof(uint32_t) * slices * c.batch, 256);
        w.tmax_stride = tile_stride(c);
        w.total = align_up(w.tmax_off + sizeof(uint32_t) * w.tmax_stride * c.batch, 256);
        return w;
    }
    const size_t slices = (size_t)topk_slices(c);
    const size_t cand = slices > 1 ? sizeof(uint32_t) * 2 * cand_stride(c, k) * c.batch : 0;
    w.cand2_off = align_up(w.cand_off + cand, 256);
    const size_t cand2 = topk_groups(c, k) > 0 ? sizeof(uint2) * cand2_stride(c, k) * c.batch : 0;
    w.total = align_up(w.cand2_off + cand2, 256);
    return w;
}

PoolWorkspace pool_workspace(const cskv_cache &c, int k, int pool_blocks, int block)
{
    PoolWorkspace w;
    const size_t items = ((size_t)c.capacity + block - 1) / block;
    w.bkey_stride = (items + 63) / 64 * 64;
    w.bslices = (int)((items + kSliceKeys - 1) / kSliceKeys);
    w.bcand_stride = ((size_t)w.bslices * pool_blocks + 1) & ~(size_t)1;
    w.bkeys_off = topk_workspace(c, k).total;
    w.bcand_off = align_up(w.bkeys_off + sizeof(uint32_t) * w.bkey_stride * c.batch, 256);
    w.build_total = align_up(w.bcand_off + (w.bslices > 1 ? sizeof(uint2) * w.bcand_stride * c.batch : 0), 256);
    w.inpool_total = align_up(sizeof(uint2) * (size_t)pool_blocks * block * c.batch, 256);
    return w;
}

namespace {

// ---------------------------------------------------------------- select

constexpr int kBins = 2048;
constexpr int kDigit = 11;
constexpr int kSliceThreads = 512;                      // slice blocks of kSliceKeys keys: 8 waves
constexpr int kMergeThreads = 512;                      // merge blocks: 8 waves
constexpr int kMergePerSmall = 10;                      // up to 5120 candidates in one round
constexpr int kMergePer = 36;                           // more: 18432 per round

// Items of one selection, in ascending index order: a contiguous key array
// (the item at position p has index base + p; positions < n are valid), or
// the concatenated candidate lists of the slices of one sequence (k (key,
// index) pairs per slice; unused slots hold key 0 and are never valid).
// Key 0 is the key of a score whose bits are all ones (a NaN), which the
// scan cannot produce from finite inputs.
struct Items {
    const uint32_t *keys;   // contiguous mode
    const uint2 *pairs;     // list mode
    int64_t n;              // positions
    int64_t base;           // contiguous mode: index of position 0
};

struct SelectArgs {
    const uint32_t *keys;   // [B][key_stride]
    uint2 *cand;            // [B][cand_stride]: slices x k (key, index) pairs per sequence
    const int32_t *n_tokens;
    int32_t *out;           // [B][k]
    int capacity, k, slices;
    size_t key_stride, cand_stride;
    int group;              // entries per item: a sequence of E entries has ceil(E / group) items
    int ratio;              // tokens per entry of the cache
    int slice_keys = kSliceKeys;  // keys per slice (the kernels' KEYS)
    // two-level merge (groups > 0): the group lists [B][cand2_stride],
    // groups x k (key, index) pairs per sequence
    uint2 *cand2 = nullptr;
    size_t cand2_stride = 0;
    int groups = 0;
    // bound select (caches the tile select serves): the largest key of every
    // 16-entry tile [B][tmax_stride]; the slices' candidate counts [B][slices]
    const uint32_t *tmax = nullptr;
    size_t tmax_stride = 0;
    uint32_t *tcount = nullptr;
};

// Items of sequence b: its entries, or its blocks of `group` entries.
__device__ __forceinline__ int64_t items_of(const SelectArgs &a, int b)
{
    return (entries_of(a.n_tokens, b, a.capacity, a.ratio) + a.group - 1) / a.group;
}

template <int THREADS>
struct SelectSmem {
    static constexpr int kWaves = THREADS / kWave;
    uint32_t bins[kBins];
    uint32_t wave_sum[kWaves];
    uint32_t red[4][kWaves];
    uint32_t found[3];
};

// Inclusive prefix sum over the block; *total receives the block sum.
template <int THREADS>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *wave_sum, uint32_t *total)
{
    constexpr int kWaves = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    v = wave_scan_add(v);
    if (lane == kWave - 1) wave_sum[w] = v;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t x = wave_sum[i];
        base += i < w ? x : 0u;
        tot += x;
    }
    *total = tot;
    __syncthreads();
    return v + base;
}

// Over the histogram in sm.bins (nbins <= 2048), the highest bin t with
// (count above t) < need <= (count at or above t); sm.found = {t, count
// strictly above t, count in t}.  Run by wave 0 alone: lane l owns the 32
// bins below nbins - 32 l (read in a rotated order so that no two lanes hit
// one LDS bank); a lane prefix sum and a ballot name the group that holds
// the threshold, then lanes 0..31 take that group's bins from the top and a
// second prefix sum and ballot name the bin.  Afterwards every bin is
// cleared for the next histogram.  Requires need <= total count.
template <class Smem>
__device__ __forceinline__ void find_threshold_bin_wave0(Smem &sm, int nbins, uint32_t need)
{
    constexpr int kOwn = kBins / kWave;           // 32 bins per lane
    const int lane = threadIdx.x;
    const int top = nbins - 1 - kOwn * lane;      // this lane's highest bin
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kOwn; ++j) {
        const int bn = top - ((j + lane) & (kOwn - 1));
        sum += bn >= 0 ? sm.bins[bn] : 0u;
    }
    const uint32_t incl = wave_scan_add(sum);
    const int owner = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
    const uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), owner);
    const int otop = nbins - 1 - kOwn * owner;
    const uint32_t c = (lane < kOwn && otop - lane >= 0) ? sm.bins[otop - lane] : 0u;
    const uint32_t ci = wave_scan_add(c);
    const int j = __ffsll((unsigned long long)__ballot(lane < kOwn && run + ci >= need)) - 1;
    if (lane == j) {
        sm.found[0] = (uint32_t)(otop - j);
        sm.found[1] = run + ci - c;
        sm.found[2] = c;
    }
#pragma unroll
    for (int jj = 0; jj < kOwn; ++jj) sm.bins[kOwn * lane + ((jj + lane) & (kOwn - 1))] = 0u;
}

// The keys of positions [PER t, PER t + PER) of round r, held by thread t,
// and their validity bits (list mode: a position past n or a slot holding
// key 0 is not valid).  Every load is issued before any is waited for (a
// position past n reads position 0 instead, and is masked): a contiguous
// array is read 16 bytes at a time and must be readable up to n rounded up
// to a multiple of 4 (every key array here is padded to 64 per sequence);
// lists are read one pair at a time.
template <bool kList, int THREADS, int PER>
__device__ __forceinline__ uint64_t load_keys(const Items &it, int64_t r, uint32_t (&key)[PER],
                                              uint32_t (&idx)[PER])
{
    const int64_t p0 = r * (int64_t)(THREADS * PER) + (int64_t)PER * threadIdx.x;
    const int64_t nv = it.n - p0;
    const uint64_t vm = nv >= PER ? (PER == 64 ? ~0ull : (1ull << PER) - 1ull) : (nv > 0 ? (1ull << nv) - 1ull : 0ull);
    if constexpr (!kList) {
        static_assert(PER % 4 == 0, "contiguous keys load as uint4");
#pragma unroll
        for (int i = 0; i < PER; i += 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(it.keys + (i < nv ? p0 + i : 0));
            key[i] = v.x; key[i + 1] = v.y; key[i + 2] = v.z; key[i + 3] = v.w;
        }
        return vm;
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint2 u = it.pairs[i < nv ? p0 + i : 0];
            key[i] = u.x;
            idx[i] = u.y;
        }
        uint64_t lv = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) lv |= (uint64_t)(key[i] != 0u) << i;
        return vm & lv;
    }
}

// Where the k-th largest valid key of `it` lies: items with key >> tshift
// greater than T are among the k largest, and of those with key >> tshift ==
// T the first `ties` in index order complete the set.  `it` holds at least k
// valid items.  Thread t holds PER consecutive positions of each round in
// key / idx (loaded here when there are several rounds).
struct Threshold {
    uint32_t T;
    int tshift;
    uint32_t ties;
};

// max_passes limits the histogram passes: when it stops the search early,
// T << tshift is still a lower bound of the k-th largest key (that key has
// prefix T at shift tshift).
template <bool kList, int THREADS, int PER>
__device__ __forceinline__ Threshold radix_threshold(SelectSmem<THREADS> &sm, const Items &it, int k,
                                                     uint32_t (&key)[PER], uint32_t (&idx)[PER], uint64_t &vm,
                                                     int64_t rounds, int max_passes = 64)
{
    constexpr int kWaves = THREADS / kWave;
    const int t = threadIdx.x;
    // ---- range of the valid keys, and the bits in which any two differ
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, orv = 0u, andv = 0xFFFFFFFFu;
    for (int64_t r = 0; r < rounds; ++r) {
        if (rounds > 1) vm = load_keys<kList, THREADS, PER>(it, r, key, idx);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool v = (vm >> i) & 1ull;
            lo = min(lo, v ? key[i] : 0xFFFFFFFFu);
            hi = max(hi, v ? key[i] : 0u);
            orv |= v ? key[i] : 0u;
            andv &= v ? key[i] : 0xFFFFFFFFu;
        }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    orv = wave_or_u32(orv);
    andv = wave_and_u32(andv);
    if ((t & (kWave - 1)) == 0) {
        sm.red[0][t / kWave] = lo;
        sm.red[1][t / kWave] = hi;
        sm.red[2][t / kWave] = orv;
        sm.red[3][t / kWave] = andv;
    }
    for (int i = t; i < kBins; i += THREADS) sm.bins[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        lo = min(lo, sm.red[0][i]);
        hi = max(hi, sm.red[1][i]);
        orv |= sm.red[2][i];
        andv &= sm.red[3][i];
    }
    // bits below `low` are the same in every valid key: they never split a tie
    const uint32_t vary = orv ^ andv;
    const int low = vary ? __builtin_ctz(vary) : 0;

    // ---- radix passes: digit windows below the common prefix of lo and hi,
    // down to bit `low`.  After a pass, items whose key >> shift exceeds the
    // threshold prefix are in; if the threshold bin is taken whole, it is in
    // too and the search stops; otherwise the bin is refined by the next
    // lower bits.  At shift `low` the prefix identifies the k-th largest key
    // itself.
    uint32_t T = lo;                 // selected: key >> tshift > T, or == T within the tie quota
    int tshift = 0;
    uint32_t ties = (uint32_t)k;
    if (lo != hi) {
        const int top = 32 - __clz((int)(lo ^ hi));      // bits [low, top) vary
        int shift = top - kDigit > low ? top - kDigit : low;
        uint32_t sub = lo >> shift;                      // first window: offset from lo
        int pshift = 32;
        uint32_t prefix = 0;
        uint32_t mask = kBins - 1;
        uint32_t need = (uint32_t)k;
        while (true) {
            const int nbins = pshift >= 32 ? kBins : 1 << (pshift - shift);
            for (int64_t r = 0; r < rounds; ++r) {
                if (rounds > 1) vm = load_keys<kList, THREADS, PER>(it, r, key, idx);
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const uint32_t x = key[i];
                    if (((vm >> i) & 1ull) && (pshift >= 32 || (x >> (pshift & 31)) == prefix))
                        atomicAdd(&sm.bins[((x >> shift) - sub) & mask], 1u);
                }
            }
            __syncthreads();
            if (t < kWave) find_threshold_bin_wave0(sm, nbins, need);
            __syncthreads();
            const uint32_t bin = sm.found[0], a2 = sm.found[1], cnt = sm.found[2];
            // key >> shift of the threshold key
            prefix = pshift >= 32 ? bin + sub : (prefix << (pshift - shift)) | bin;
            need -= a2;
            if (shift == low || cnt == need || --max_passes == 0) {
                T = prefix;
                tshift = shift;
                ties = need;
                break;
            }
            pshift = shift;
            shift = shift - kDigit > low ? shift - kDigit : low;
            sub = 0;
            mask = (1u << (pshift - shift)) - 1u;
        }
    }
    return Threshold{T, tshift, ties};
}

// Exact top-k of `it`, which holds more than k valid items.  Thread t holds
// PER consecutive positions in registers.  kPairsOut: write the selected
// (key, index) pairs in index order; else the indices.  Exactly k items are
// selected, so nothing is padded.
template <bool kList, bool kPairsOut, int THREADS, int PER>
__device__ __forceinline__ void select_topk(SelectSmem<THREADS> &sm, const Items &it, int k, int32_t *out_idx,
                            uint2 *out_pairs)
{
    constexpr int kRound = THREADS * PER;
    const int t = threadIdx.x;
    const int64_t rounds = (it.n + kRound - 1) / kRound;
    uint32_t key[PER], idx[PER];
    uint64_t vm = 0;
    if (rounds == 1) vm = load_keys<kList, THREADS, PER>(it, 0, key, idx);
    const Threshold th = radix_threshold<kList, THREADS, PER>(sm, it, k, key, idx, vm, rounds);
    const uint32_t T = th.T, ties = th.ties;
    const int tshift = th.tshift;
    // Items with key >> tshift == T: the first `ties` of them in index order
    // complete the set (all of them when the bin was taken whole).

    // ---- ordered emission
    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t r = 0; r < rounds; ++r) {
        if (rounds > 1) vm = load_keys<kList, THREADS, PER>(it, r, key, idx);
        const int64_t p0 = r * (int64_t)kRound + (int64_t)PER * t;
        uint64_t gtm = 0, eqm = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool v = (vm >> i) & 1ull;
            const uint32_t xs = key[i] >> tshift;
            gtm |= (uint64_t)(v && xs > T) << i;
            eqm |= (uint64_t)(v && xs == T) << i;
        }
        const uint32_t ngt = __popcll(gtm), neq = __popcll(eqm);
        uint32_t tot;
        const uint32_t mine = (ngt << 16) | neq;
        const uint32_t excl = block_scan<THREADS>(mine, sm.wave_sum, &tot) - mine;
        // Tied items take the remaining tie slots in index order.  (Written
        // with a running rank and a comparison: a form with an unsigned
        // saturating difference was mis-lowered by the compiler.)
        uint32_t eqr = eq_base + (excl & 0xFFFFu);
        uint32_t pos = gt_base + (excl >> 16) + min(eqr, ties);
        if (gtm | eqm) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const bool g = (gtm >> i) & 1ull, q = (eqm >> i) & 1ull;
                if (g || q) {
                    bool sel = true;
                    if (q) {
                        sel = eqr < ties;
                        ++eqr;
                    }
                    if (sel) {
                        if (pos < (uint32_t)k) {
                            const uint32_t ix = kList ? idx[i] : (uint32_t)(it.base + p0 + i);
                            if (kPairsOut) out_pairs[pos] = make_uint2(key[i], ix);
                            else out_idx[pos] = (int32_t)ix;
                        }
                        ++pos;
                    }
                }
            }
        }
        gt_base += tot >> 16;
        eq_base += tot & 0xFFFFu;
    }
}

// Sequence b longer than one slice, slice s: the local top-k of keys
// [s*KEYS, (s+1)*KEYS) as index-ordered (key, index) pairs; a
// slice with at most k entries passes them all and pads its list with key 0.
// The slices' lists contain the sequence's top-k (an entry beaten by fewer
// than k entries overall is beaten by fewer than k in its slice).
template <int KEYS, int THREADS>
__global__ __launch_bounds__(THREADS) void topk_slice_kernel(SelectArgs a)
{
    __shared__ SelectSmem<THREADS> sm;
    const int b = blockIdx.y, s = blockIdx.x;
    const int64_t E = items_of(a, b);
    if (E <= a.k || E <= KEYS) return;         // the merge reads the keys directly
    uint2 *out = a.cand + (size_t)b * a.cand_stride + (size_t)s * a.k;
    const int64_t first = (int64_t)s * KEYS;
    if (first >= E) return;
    const int64_t n = E - first < KEYS ? E - first : KEYS;
    if (n <= a.k) {
        for (int i = threadIdx.x; i < a.k; i += THREADS)
            out[i] = i < n ? make_uint2(a.keys[(size_t)b * a.key_stride + first + i], (uint32_t)(first + i))
                           : make_uint2(0u, 0xFFFFFFFFu);
        return;
    }
    Items it{a.keys + (size_t)b * a.key_stride + first, nullptr, n, first};
    select_topk<false, true, THREADS, KEYS / THREADS>(sm, it, a.k, nullptr, out);
}

// Sequence b of a cache that fits one slice: the final top-k from the key
// array.
template <int KEYS, int THREADS>
__global__ __launch_bounds__(THREADS) void topk_select_kernel(SelectArgs a)
{
    __shared__ SelectSmem<THREADS> sm;
    const int b = blockIdx.x;
    const int64_t E = items_of(a, b);
    int32_t *out = a.out + (size_t)b * a.k;
    if (E <= a.k) {
        for (int i = threadIdx.x; i < a.k; i += THREADS) out[i] = i < E ? i : -1;
        return;
    }
    Items it{a.keys + (size_t)b * a.key_stride, nullptr, E, 0};
    select_topk<false, false, THREADS, KEYS / THREADS>(sm, it, a.k, out, nullptr);
}

// Bound select, first kernel: the slices of sequence b (blocks of THREADS
// threads, KEYS keys per slice).  The bound V is the prefix bin, after one
// histogram pass over the sequence's group maxima (the largest key of each
// group of consecutive 16-entry tiles), that holds the k-th largest of them
// (every key when there are at most k groups): at least k groups hold a
// key >= V, so the sequence's k largest keys are all >= V.  A slice's keys
// >= V go to its candidate list as (key, index) pairs in index order, with
// their count.
//
// A group is the fewest tiles that fit the sequence's tile maxima in one
// block, 16 groups per thread: 1 tile up to 131,072 entries, then 2, then
// up to G.  A sequence gets min(slices, max(32, 512 / batch)) blocks; block
// x handles slices x, x + gridDim.x, ... that hold entries.  Its first
// slice's keys and the ungrouped tile maxima are read at once with the
// entry count, bounded by the capacity and masked by the entries when they
// arrive, so a block of a sequence that fits ungrouped waits for memory
// once; blocks past the entries leave.

// Group maxima of thread t (groups 16 t .. 16 t + 15 of G tiles each, 0 for
// groups past the entries) and the bound V from them.
template <int THREADS, int G>
__device__ __forceinline__ uint32_t bound_from_groups(SelectSmem<THREADS> &sm, const SelectArgs &a, int b,
                                                      const uint32_t (&tl)[16 * G], uint64_t tlvm, int64_t nt)
{
    constexpr int kTPer = 16;
    const int t = threadIdx.x;
    {                                              // tiles past the entries hold stale data
        const int64_t tv = nt - (int64_t)kTPer * G * t;
        tlvm &= tv >= kTPer * G ? ~0ull : (tv > 0 ? (1ull << tv) - 1ull : 0ull);
    }
    uint32_t tm[kTPer], tidx[kTPer];
    uint64_t tvm = 0;
#pragma unroll
    for (int j = 0; j < kTPer; ++j) {
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < G; ++i) m = max(m, ((tlvm >> (G * j + i)) & 1ull) ? tl[G * j + i] : 0u);
        tm[j] = m;
        tvm |= (uint64_t)((tlvm >> (G * j)) & 1ull) << j;   // a group holds entries iff its first tile does
    }
    const int64_t ng = (nt + G - 1) / G;          // groups holding entries
    if (ng <= a.k) return 0u;                      // every key is a candidate
    const Items ti{nullptr, nullptr, ng, 0};       // one round: the maxima are in registers
    const Threshold th = radix_threshold<false, THREADS, kTPer>(sm, ti, a.k, tm, tidx, tvm, 1, 1);
    __syncthreads();                               // sm is used again afterwards
    return th.T << th.tshift;
}

// The keys >= V of slice s (keys already loaded, kvm masked to its entries)
// to the slice's candidate list, with their count.
template <int KEYS, int THREADS>
__device__ __forceinline__ void bound_candidates(SelectSmem<THREADS> &sm, const SelectArgs &a, int b, int s,
                                                 const uint32_t (&key)[KEYS / THREADS], uint64_t kvm, uint32_t V)
{
    constexpr int PER = KEYS / THREADS;
    const int t = threadIdx.x;
    uint32_t in = 0, mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool c = ((kvm >> i) & 1ull) && key[i] >= V;
        in |= (uint32_t)c << i;
        mine += c;
    }
    uint32_t total;
    uint32_t pos = block_scan<THREADS>(mine, sm.wave_sum, &total) - mine;
    uint2 *out = a.cand + (size_t)b * a.cand_stride + (size_t)s * KEYS;
    const int64_t p0 = (int64_t)s * KEYS + (int64_t)PER * t;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if ((in >> i) & 1u) out[pos++] = make_uint2(key[i], (uint32_t)(p0 + i));
    if (t == 0) a.tcount[(size_t)b * a.slices + s] = total;
}

// V from groups of GS tiles, read after the entry count.
template <int THREADS, int GS>
__device__ __forceinline__ uint32_t bound_grouped(SelectSmem<THREADS> &sm, const SelectArgs &a, int b, int64_t nt)
{
    static_assert(16 * GS <= 64, "tile maxima per thread");
    const Items tit{a.tmax + (size_t)b * a.tmax_stride, nullptr, nt, 0};
    uint32_t tl[16 * GS], tlidx[16 * GS];
    const uint64_t tlvm = load_keys<false, THREADS, 16 * GS>(tit, 0, tl, tlidx);
    return bound_from_groups<THREADS, GS>(sm, a, b, tl, tlvm, nt);
}

// Block x of nx of sequence b.
template <int KEYS, int THREADS, int G>
__device__ __forceinline__ void bound_slice(SelectSmem<THREADS> &sm, const SelectArgs &a, int x, int nx, int b)
{
    constexpr int PER = KEYS / THREADS;
    constexpr int kTPer = 16;
    const int t = threadIdx.x;
    const int64_t first = (int64_t)x * KEYS;
    const int64_t ncap = a.capacity - first < KEYS ? a.capacity - first : KEYS;
    uint32_t key[PER], kidx[PER];
    uint64_t kvm;
    {
        const Items kit{a.keys + (size_t)b * a.key_stride + first, nullptr, ncap, first};
        kvm = load_keys<false, THREADS, PER>(kit, 0, key, kidx);
    }
    const Items tit{a.tmax + (size_t)b * a.tmax_stride, nullptr, (a.capacity + 15) / 16, 0};
    uint32_t tl[kTPer], tlidx[kTPer];
    const uint64_t tlvm = load_keys<false, THREADS, kTPer>(tit, 0, tl, tlidx);
    const int64_t E = items_of(a, b);
    if (E <= a.k || first >= E) return;           // the final kernel pads or reads only used slices
    {                                              // positions past the entries hold stale data
        const int64_t kv = (E - first < KEYS ? E - first : KEYS) - (int64_t)PER * t;
        kvm &= kv >= PER ? ~0ull : (kv > 0 ? (1ull << kv) - 1ull : 0ull);
    }
    const int64_t nt = (E + 15) / 16;
    uint32_t V;
    if (G == 1 || nt <= kTPer * THREADS)
        V = bound_from_groups<THREADS, 1>(sm, a, b, tl, tlvm, nt);
    else if (G == 2 || nt <= 2 * kTPer * THREADS)
        V = bound_grouped<THREADS, (G > 2 ? 2 : G)>(sm, a, b, nt);
    else
        V = bound_grouped<THREADS, G>(sm, a, b, nt);
    for (int s = x;;) {
        bound_candidates<KEYS, THREADS>(sm, a, b, s, key, kvm, V);
        s += nx;
        if ((int64_t)s * KEYS >= E) break;
        __syncthreads();                           // sm.wave_sum is used again
        const int64_t f = (int64_t)s * KEYS;
        const Items kit{a.keys + (size_t)b * a.key_stride + f, nullptr, E - f < KEYS ? E - f : KEYS, f};
        kvm = load_keys<false, THREADS, PER>(kit, 0, key, kidx);
    }
}

template <int KEYS, int THREADS, int G>
__global__ __launch_bounds__(THREADS) void topk_bound_slice_kernel(SelectArgs a)
{
    __shared__ SelectSmem<THREADS> sm;
    bound_slice<KEYS, THREADS, G>(sm, a, blockIdx.x, gridDim.x, blockIdx.y);
}

// The slice launch of a decode step that carries its deferred entry: plane
// z = 0 of the grid holds the slice blocks; the blocks of the planes after
// it hold the compressor's waves (compress_wave_slots: 2 channels by two
// groups of 4 rows each, nx x ceil(batch / 8) of them), taken in order, 8 to
// a block.  A
// block's kind follows from its index alone, so the slice blocks issue their
// loads without waiting for an argument first.  The two kinds share no data.  Two blocks fit a CU (at most 128
// registers a lane), so the compressor's blocks run beside the slice blocks
// rather than after them.  Measured against 5 channels a wave, against
// blocks that stage 8 rows in LDS for 16 channels and against one, three or
// four row groups a wave, this shape adds the least to the launch on the
// steps that complete entries (about 2 us at 64K x 32: its 144 blocks and the
// 288 slice blocks run in one round of two blocks a CU).
constexpr int kCarryRows = 4, kCarryCpw = 2, kCarryGroups = 2, kCarryWaves = kSliceThreads / kWave;
constexpr int kCarryMaxBatch = 64;

// What the carried compressor and quantiser read, and nothing more: kernel
// arguments are copied into every launch's argument buffer and loaded by its
// waves, and the full descriptors made both carrying launches measurably
// slower (624 argument bytes against 128).
struct CarriedEntry {
    const float *tokens, *w_comp, *pending;
    float *ent;
    int64_t *slots;
    uint8_t *k_codes, *v_codes;
    float *k_scales, *v_scales;
    int32_t batch, dim, rope_dim, k_group, v_group, k_format;
};

__device__ __forceinline__ AppendArgs append_args_of(const CarriedEntry &e)
{
    AppendArgs d{};
    d.c.batch = e.batch;
    d.c.dim = e.dim;
    d.c.rope_dim = e.rope_dim;
    d.c.k_group = e.k_group;
    d.c.v_group = e.v_group;
    d.c.k_format = e.k_format;
    d.c.k_codes = e.k_codes;
    d.c.k_scales = e.k_scales;
    d.c.v_codes = e.v_codes;
    d.c.v_scales = e.v_scales;
    d.c.pending = const_cast<float *>(e.pending);
    d.tokens = e.tokens;
    d.w_comp = e.w_comp;
    d.ent = e.ent;
    d.total_new = e.batch;
    d.slots = e.slots;
    return d;
}

struct CarriedCompress {
    CarriedEntry e;
    int nx, waves;
};

template <int KEYS, int THREADS, int G>
__global__ __launch_bounds__(THREADS, 2 * THREADS / 256) void topk_bound_slice_carry_kernel(SelectArgs a,
                                                                                           CarriedCompress cc)
{
    static_assert(THREADS == kCarryWaves * kWave, "the compressor's block shape");
    __shared__ SelectSmem<THREADS> sm;
    if (blockIdx.z == 0) {
        bound_slice<KEYS, THREADS, G>(sm, a, blockIdx.x, gridDim.x, blockIdx.y);
        return;
    }
    const int cb = (((int)blockIdx.z - 1) * (int)gridDim.y + (int)blockIdx.y) * (int)gridDim.x + (int)blockIdx.x;
    const int wi = cb * kCarryWaves + (int)(threadIdx.x / kWave);
    if (wi < cc.waves)
        compress_wave_slots<kCarryRows, kCarryCpw, kCarryGroups>(append_args_of(cc.e), wi % cc.nx, wi / cc.nx);
}

// Bound select, second kernel: sequence b's candidate lists (slice order is
// index order) gathered into LDS, then the exact top-k among them; more
// candidates than kFinalCap (heavily tied scores at the bound) select over
// every key of the sequence instead.  The entry count, the slices' counts
// (MAXS slices at most) and the first pairs of every slice are read at
// once: 4096 / MAXS pairs of each slice and, past 32 slices, 128 more of
// each of the first 32 (few long slices and many short ones both fit); the
// pairs past those, if any, are read afterwards, all at once.
constexpr int kFinalThreads = 512;
constexpr int kFinalPer = 12;
constexpr int kFinalCap = kFinalThreads * kFinalPer;
constexpr int kSpec = 128, kSpecSlices = 32;
template <int MAXS>
struct FinalSmem {
    SelectSmem<kFinalThreads> sm;
    alignas(16) uint2 lc[kFinalCap];
    uint32_t pre[MAXS + 1];
};

template <int MAXS>
__device__ __forceinline__ void bound_final(FinalSmem<MAXS> &f, const SelectArgs &a, int b)
{
    static_assert(MAXS <= kFinalThreads && MAXS >= kSpecSlices, "one slice count per thread");
    constexpr int kA = 4096 / MAXS;                // pairs of every slice
    constexpr int kB = MAXS > kSpecSlices ? kSpec : 0;   // more pairs of the first kSpecSlices
    constexpr int kSpecPer = 4096 / kFinalThreads, kSpecPerB = kB ? kSpecSlices * kB / kFinalThreads : 0;
    auto covered = [](int sl) { return (uint32_t)(kA + (sl < kSpecSlices ? kB : 0)); };
    SelectSmem<kFinalThreads> &sm = f.sm;
    uint2 *const lc = f.lc;
    uint32_t *const pre = f.pre;
    const int t = threadIdx.x;
    const uint2 *cl = a.cand + (size_t)b * a.cand_stride;
    // speculative reads, unused for slices past the entries or the capacity
    uint2 sp[kSpecPer], spb[kSpecPerB ? kSpecPerB : 1];
#pragma unroll
    for (int i = 0; i < kSpecPer; ++i) {
        const int u = t + kFinalThreads * i, sl = u / kA, j = u % kA;
        sp[i] = cl[(size_t)(sl < a.slices ? sl : 0) * kSliceKeys + j];
    }
#pragma unroll
    for (int i = 0; i < kSpecPerB; ++i) {
        const int u = t + kFinalThreads * i, sl = u / kSpec, j = kA + u % kSpec;
        spb[i] = cl[(size_t)(sl < a.slices ? sl : 0) * kSliceKeys + j];
    }
    const uint32_t cnt = t < a.slices ? a.tcount[(size_t)b * a.slices + t] : 0u;
    const int64_t E = items_of(a, b);
    int32_t *out = a.out + (size_t)b * a.k;
    if (E <= a.k) {
        for (int i = t; i < a.k; i += kFinalThreads) out[i] = i < E ? i : -1;
        return;
    }
    const int used = (int)((E + kSliceKeys - 1) / kSliceKeys);
    {                                              // prefix of the used slices' counts
        const uint32_t c = t < used ? cnt : 0u;
        uint32_t tot;
        const uint32_t incl = block_scan<kFinalThreads>(c, sm.wave_sum, &tot);
        if (t <= used) pre[t] = incl - c;
    }
    const bool spill = __syncthreads_or(t < used && cnt > covered(t));
    const uint32_t total = pre[used];
    if (total > (uint32_t)kFinalCap) {
        const Items it{a.keys + (size_t)b * a.key_stride, nullptr, E, 0};
        select_topk<false, false, kFinalThreads, 8>(sm, it, a.k, out, nullptr);
        return;
    }
#pragma unroll
    for (int i = 0; i < kSpecPer; ++i) {
        const int u = t + kFinalThreads * i, sl = u / kA, j = u % kA;
        if (sl < used && (uint32_t)j < pre[sl + 1] - pre[sl]) lc[pre[sl] + j] = sp[i];
    }
#pragma unroll
    for (int i = 0; i < kSpecPerB; ++i) {
        const int u = t + kFinalThreads * i, sl = u / kSpec, j = kA + u % kSpec;
        if (sl < used && (uint32_t)j < pre[sl + 1] - pre[sl]) lc[pre[sl] + j] = spb[i];
    }
    if (spill) {                                   // pairs the speculative reads left out
        uint2 rest[kFinalPer];
        uint32_t need = 0;
#pragma unroll
        for (int i = 0; i < kFinalPer; ++i) {
            const uint32_t p = t + kFinalThreads * i;
            int sl = 0;                            // the last slice whose list starts at or before p
#pragma unroll
            for (int w = MAXS / 2; w > 0; w >>= 1)
                if (sl + w < used && pre[sl + w] <= p) sl += w;
            const uint32_t j = p - pre[sl];
            const bool r = p < total && j >= covered(sl);
            rest[i] = cl[(size_t)sl * kSliceKeys + (r ? j : 0u)];
            need |= (uint32_t)r << i;
        }
#pragma unroll
        for (int i = 0; i < kFinalPer; ++i)
            if ((need >> i) & 1u) lc[t + kFinalThreads * i] = rest[i];
    }
    __syncthreads();
    if (total == (uint32_t)a.k) {                  // exactly the k largest
        for (int i = t; i < a.k; i += kFinalThreads) out[i] = (int32_t)lc[i].y;
        return;
    }
    // the select's work grows with its item slots: few candidates take few
    const Items it{nullptr, lc, (int64_t)total, 0};
    if (total <= (uint32_t)(kFinalThreads * 2))
        select_topk<true, false, kFinalThreads, 2>(sm, it, a.k, out, nullptr);
    else
        select_topk<true, false, kFinalThreads, kFinalPer>(sm, it, a.k, out, nullptr);
}

template <int MAXS>
__global__ __launch_bounds__(kFinalThreads) void topk_bound_final_kernel(SelectArgs a)
{
    __shared__ FinalSmem<MAXS> f;
    bound_final<MAXS>(f, a, blockIdx.x);
}

// The final launch of a decode step that carries its deferred entry: block
// (b, 0) selects for sequence b, block (b, 1) quantises its compressed entry
// (if the head recorded one) into its cache row, before attention reads it.
template <int MAXS>
__global__ __launch_bounds__(kFinalThreads) void topk_bound_final_carry_kernel(SelectArgs a, CarriedEntry e)
{
    static_assert(kFinalThreads == 512, "quantize_main_512 takes the entry on 512 threads");
    __shared__ FinalSmem<MAXS> f;
    const int b = blockIdx.x;
    if (blockIdx.y == 0) {
        bound_final<MAXS>(f, a, b);
        return;
    }
    const int64_t slot = e.slots[b];
    if (slot >= 0)
        quantize_main_512(append_args_of(e), e.ent + (size_t)b * kDim, threadIdx.x, (size_t)slot,
                          reinterpret_cast<float *>(f.sm.bins));
}

// Sequence b of a cache whose capacity spans several slices: the final top-k
// over the slices' candidate lists (index-ordered, so their concatenation is
// too), or straight from the key array when the sequence fits one slice.
template <int KEYS>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(SelectArgs a)
{
    __shared__ SelectSmem<kMergeThreads> sm;
    const int b = blockIdx.x;
    const int64_t E = items_of(a, b);
    int32_t *out = a.out + (size_t)b * a.k;
    if (E <= a.k) {
        for (int i = threadIdx.x; i < a.k; i += kMergeThreads) out[i] = i < E ? i : -1;
        return;
    }
    if (E <= KEYS) {
        Items it{a.keys + (size_t)b * a.key_stride, nullptr, E, 0};
        select_topk<false, false, kMergeThreads, KEYS / kMergeThreads>(sm, it, a.k, out, nullptr);
        return;
    }
    // every list is full but the last slice's, whose first min(k, its
    // entries) slots are valid: the padding after them is not read
    const int64_t used = (E + KEYS - 1) / KEYS;
    const int64_t last = E - (used - 1) * KEYS;
    if (a.groups > 0) {
        // the group lists: a group of two or more slices holds exactly k
        // valid pairs (its first slice is full, k < 4096), a one-slice
        // group its slice's list (pads hold key 0, never valid)
        const int64_t ug = (used + kGroupSlices - 1) / kGroupSlices;
        const uint2 *gl = a.cand2 + (size_t)b * a.cand2_stride;
        if (ug == 1) {                              // group 0 has >= 2 slices: its k pairs are the answer
            for (int i = threadIdx.x; i < a.k; i += kMergeThreads) out[i] = (int32_t)gl[i].y;
            return;
        }
        Items it{nullptr, gl, ug * a.k, 0};
        if (it.n <= kMergeThreads * kMergePerSmall)
            select_topk<true, false, kMergeThreads, kMergePerSmall>(sm, it, a.k, out, nullptr);
        else
            select_topk<true, false, kMergeThreads, kMergePer>(sm, it, a.k, out, nullptr);
        return;
    }
    Items it{nullptr, a.cand + (size_t)b * a.cand_stride, (used - 1) * a.k + (last < a.k ? last : a.k), 0};
    if (it.n <= kMergeThreads * kMergePerSmall)
        select_topk<true, false, kMergeThreads, kMergePerSmall>(sm, it, a.k, out, nullptr);
    else
        select_topk<true, false, kMergeThreads, kMergePer>(sm, it, a.k, out, nullptr);
}

// First level of the two-level merge: group g of sequence b, slices
// [8 g, 8 g + 8) of those holding entries, to its top-k (key, index) pairs
// in index order.  The union of the groups' top-k lists holds the
// sequence's top-k, as the slices' lists do.
template <int KEYS>
__global__ __launch_bounds__(kMergeThreads) void topk_group_kernel(SelectArgs a)
{
    __shared__ SelectSmem<kMergeThreads> sm;
    const int b = blockIdx.y, g = blockIdx.x;
    const int64_t E = items_of(a, b);
    if (E <= a.k || E <= KEYS) return;         // the merge reads the keys directly
    const int64_t used = (E + KEYS - 1) / KEYS;
    const int64_t s0 = (int64_t)g * kGroupSlices;
    if (s0 >= used) return;                          // the merge reads only the groups in use
    const int64_t s1 = s0 + kGroupSlices < used ? s0 + kGroupSlices : used;
    uint2 *out = a.cand2 + (size_t)b * a.cand2_stride + (size_t)g * a.k;
    const uint2 *in = a.cand + (size_t)b * a.cand_stride + (size_t)s0 * a.k;
    if (s1 - s0 == 1) {                              // one list: its own top-k already
        for (int i = threadIdx.x; i < a.k; i += kMergeThreads) out[i] = in[i];
        return;
    }
    // the group's first slice is full (4096 > k entries): more than k valid
    const int64_t last = s1 == used ? E - (used - 1) * KEYS : KEYS;
    Items it{nullptr, in, (s1 - s0 - 1) * a.k + (last < a.k ? last : a.k), 0};
    if (it.n <= kMergeThreads * kMergePerSmall)
        select_topk<true, true, kMergeThreads, kMergePerSmall>(sm, it, a.k, nullptr, out);
    else
        select_topk<true, true, kMergeThreads, kMergePer>(sm, it, a.k, nullptr, out);
}

// Top-k among the pooled entries of sequence b, from the pooled scan's
// (key, entry) pairs in pool order (ascending entries; key 0 = no entry).
// A sequence of at most k entries has them all in the pool.
__global__ __launch_bounds__(kMergeThreads) void topk_pool_select_kernel(SelectArgs a)
{
    __shared__ SelectSmem<kMergeThreads> sm;
    const int b = blockIdx.x;
    const int64_t E = entries_of(a.n_tokens, b, a.capacity, a.ratio);
    int32_t *out = a.out + (size_t)b * a.k;
    if (E <= a.k) {
        for (int i = threadIdx.x; i < a.k; i += kMergeThreads) out[i] = i < E ? i : -1;
        return;
    }
    Items it{nullptr, a.cand + (size_t)b * a.cand_stride, (int64_t)a.cand_stride, 0};
    if (it.n <= kMergeThreads * kMergePerSmall)
        select_topk<true, false, kMergeThreads, kMergePerSmall>(sm, it, a.k, out, nullptr);
    else
        select_topk<true, false, kMergeThreads, kMergePer>(sm, it, a.k, out, nullptr);
}

// Select (slices + merge, or one select) of the k best items per sequence.
template <int KEYS, int THREADS>
void launch_select_t(const SelectArgs &se, int batch, hipStream_t s, const TimedLaunch &tk)
{
    if (se.slices > 1) {
        launch_kernel(topk_slice_kernel<KEYS, THREADS>, dim3((unsigned)se.slices, (unsigned)batch), dim3(THREADS),
                      s, tk.start, nullptr, se);
        if (se.groups > 0)
            launch_kernel(topk_group_kernel<KEYS>, dim3((unsigned)se.groups, (unsigned)batch), dim3(kMergeThreads),
                          s, nullptr, nullptr, se);
        launch_kernel(topk_merge_kernel<KEYS>, dim3((unsigned)batch), dim3(kMergeThreads), s, nullptr, tk.stop, se);
    } else {
        launch_kernel(topk_select_kernel<KEYS, THREADS>, dim3((unsigned)batch), dim3(THREADS), s, tk.start,
                      tk.stop, se);
    }
}

// Batches of kManySeqs sequences or more fill the chip with slices several
// times over; their slices take 4-wave blocks (16 keys per thread), which
// measured faster there (ragged 256-sequence batch: 27 -> 23 us) and slower
// at 32 sequences (19.1 -> 19.8 us).
constexpr int kManySeqs = 128;
void launch_select(const SelectArgs &se, int batch, hipStream_t s, const TimedLaunch &tk)
{
    if (se.slice_keys == 2 * kSliceKeys)
        launch_select_t<2 * kSliceKeys, 2 * kSliceThreads>(se, batch, s, tk);
    else if (batch >= kManySeqs)
        launch_select_t<kSliceKeys, kSliceThreads / 2>(se, batch, s, tk);
    else
        launch_select_t<kSliceKeys, kSliceThreads>(se, batch, s, tk);
}

}  // namespace

bool topk_carries_entry(const cskv_cache &c, int k)
{
    return c.batch <= kCarryMaxBatch && topk_workspace(c, k).tiles;
}

hipError_t launch_indexer_topk(const cskv_cache &c, const uint16_t *q_idx, int heads,
                               const float *head_w, int k, int32_t *out_idx, void *ws,
                               hipStream_t s, const PoolBuild *pool, float *out_scores,
                               const DeferredEntry *entry)
{
    const TopkWorkspace lay = topk_workspace(c, k);
    if (entry && !lay.tiles) return hipErrorInvalidValue;     // only the bound select carries an entry
    uint32_t *keys = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.keys_off);
    uint2 *cand = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + lay.cand_off);
    uint32_t *bkeys = nullptr;
    PoolWorkspace pw{};
    if (pool) {
        pw = pool_workspace(c, k, pool->blocks, pool->block);
        bkeys = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pw.bkeys_off);
    }

    uint32_t *tmax = lay.tiles ? reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.tmax_off) : nullptr;
    launch_indexer_scan(c, q_idx, heads, head_w, keys, s, bkeys, pw.bkey_stride, pool ? pool->block : 1,
                        out_scores, tmax, lay.tmax_stride);

    SelectArgs se{keys, cand, c.n_tokens, out_idx, c.capacity, k, topk_slices(c), score_key_stride(c),
                  cand_stride(c, k), 1, c.ratio};
    if (lay.tiles) {
        const TimedLaunch tk = timer_take(CSKV_KERNEL_TOPK_SELECT);
        const int slices = bound_slices(c);
        se.slices = slices;
        se.cand = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + lay.tcand_off);
        se.cand_stride = (size_t)slices * kSliceKeys;
        se.tmax = tmax;
        se.tmax_stride = lay.tmax_stride;
        se.tcount = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                                 align_up(lay.tcand_off + sizeof(uint2) * se.cand_stride * c.batch, 256));
        const int per = 512 / c.batch > 32 ? 512 / c.batch : 32;
        const dim3 sg((unsigned)(slices < per ? slices : per), (unsigned)c.batch), fg((unsigned)c.batch);
        const int g = tile_group(c);
        if (entry) {
            // the step's deferred entry: compressed in the slice launch,
            // quantised in the final launch (grid rows / blocks past the
            // select's)
            const CarriedEntry d{entry->tokens, entry->w_comp, c.pending, entry->ent, entry->slots,
                                 c.k_codes, c.v_codes, c.k_scales, c.v_scales, c.batch,
                                 c.dim, c.rope_dim, c.k_group, c.v_group, c.k_format};
            const int nx = (kDim + kCarryCpw - 1) / kCarryCpw;
            constexpr int kRowsPerWave = kCarryRows * kCarryGroups;
            const CarriedCompress cc{d, nx, nx * ((c.batch + kRowsPerWave - 1) / kRowsPerWave)};
            const int blocks = (cc.waves + kCarryWaves - 1) / kCarryWaves;
            const int plane = (int)sg.x * c.batch;
            const dim3 cg(sg.x, (unsigned)c.batch, (unsigned)(1 + (blocks + plane - 1) / plane));
            auto slice_launch = [&](auto gg) {
                launch_kernel(topk_bound_slice_carry_kernel<kSliceKeys, kSliceThreads, decltype(gg)::value>, cg,
                              dim3(kSliceThreads), s, tk.start, nullptr, se, cc);
            };
            if (g == 1) slice_launch(std::integral_constant<int, 1>{});
            else if (g == 2) slice_launch(std::integral_constant<int, 2>{});
            else slice_launch(std::integral_constant<int, 4>{});
            const dim3 qg((unsigned)c.batch, 2);
            if (g == 1)
                launch_kernel(topk_bound_final_carry_kernel<32>, qg, dim3(kFinalThreads), s, nullptr, tk.stop, se, d);
            else
                launch_kernel(topk_bound_final_carry_kernel<kTileMaxCap / kSliceKeys>, qg, dim3(kFinalThreads), s,
                              nullptr, tk.stop, se, d);
        } else if (g == 1) {
            launch_kernel(topk_bound_slice_kernel<kSliceKeys, kSliceThreads, 1>, sg, dim3(kSliceThreads), s,
                          tk.start, nullptr, se);
            launch_kernel(topk_bound_final_kernel<32>, fg, dim3(kFinalThreads), s, nullptr, tk.stop, se);
        } else {
            if (g == 2)
                launch_kernel(topk_bound_slice_kernel<kSliceKeys, kSliceThreads, 2>, sg, dim3(kSliceThreads), s,
                              tk.start, nullptr, se);
            else
                launch_kernel(topk_bound_slice_kernel<kSliceKeys, kSliceThreads, 4>, sg, dim3(kSliceThreads), s,
                              tk.start, nullptr, se);
            launch_kernel(topk_bound_final_kernel<kTileMaxCap / kSliceKeys>, fg, dim3(kFinalThreads), s, nullptr,
                          tk.stop, se);
        }
    } else {
        se.slice_keys = slice_keys_of(c);
        se.groups = topk_groups(c, k);
        se.cand2 = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + lay.cand2_off);
        se.cand2_stride = cand2_stride(c, k);
        launch_select(se, c.batch, s, timer_take(CSKV_KERNEL_TOPK_SELECT));
    }
    if (pool) {
        // the pool: the best pool->blocks blocks by their largest key
        uint2 *bcand = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + pw.bcand_off);
        const SelectArgs sb{bkeys, bcand, c.n_tokens, pool->out, c.capacity, pool->blocks, pw.bslices,
                            pw.bkey_stride, pw.bcand_stride, pool->block, c.ratio};
        launch_select(sb, c.batch, s, TimedLaunch{});
    }
    return hipGetLastError();
}

hipError_t launch_indexer_topk_in_pool(const cskv_cache &c, const uint16_t *q_idx, int heads,
                                       const float *head_w, int k, const int32_t *pool, int pool_blocks,
                                       int block, int32_t *out_idx, void *ws, hipStream_t s)
{
    uint2 *pairs = static_cast<uint2 *>(ws);
    launch_pool_scan(c, q_idx, heads, head_w, pool, pool_blocks, block, pairs, s);
    const SelectArgs se{nullptr, pairs, c.n_tokens, out_idx, c.capacity, k, 1, 0,
                        (size_t)pool_blocks * block, 1, c.ratio};
    launch_kernel(topk_pool_select_kernel, dim3((unsigned)c.batch), dim3(kMergeThreads), s, nullptr, nullptr, se);
    return hipGetLastError();
}

}  // namespace cskv
