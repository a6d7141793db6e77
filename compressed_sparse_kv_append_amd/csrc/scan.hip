// scan.hip -- indexer scoring over every cached entry [P2 三、"突破四：滑动窗口和
// 稀疏注意力" (a light indexer scores all history); P2 四、"CSA2：三种模式"
// (per-layer multi-head indexer query, per-entry indexer key)].
//
// s_j = sum_h w_h * relu(q_h . K_j) is a [heads x dim] x [dim x entries]
// contraction, run on bf16 MFMA (16x16x32) with fp32 accumulation.  The keys
// plane is the only large read of the decode step, so the scan is built to
// stream it: each wave pulls 16-key tiles with coalesced, non-temporal loads
// that write straight into its own LDS ring (no registers, no block barrier),
// reads them back in the MFMA operand layout, and keeps the query in
// registers.  One round of blocks covers the chip.  The only output is one
// order-preserving uint32 key per entry, which the top-k select consumes.
//
// Hierarchical indexer [P2 "层级稀疏索引器：后面的层只在候选池里找"]: the
// scan of the layer that builds the candidate pool also writes, per block of
// `block` entries, the largest key of the block (the key order is the score
// order).  The pooled scan of a later layer reads only the rows of the
// pooled blocks -- a block's rows are contiguous -- and writes (key, entry)
// pairs in pool order, which is ascending entry order.
//
// Sources cited as [P2]:
//   P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {

namespace {

constexpr int kScanThreads = 256;   // 4 waves
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kRing = 2;            // 16-key tiles in flight per wave (LDS slots)
constexpr int kScanBlocksPerCU = 3; // blocks per CU the kernels are built for (<= 168 registers a lane)

struct ScanArgs {
    const uint16_t *keys;      // idx_keys plane
    const int32_t *n_tokens;
    const uint16_t *q;         // [B][H][Di]
    const float *head_w;       // [B][H] or null
    uint32_t *out_keys;        // [B][key_stride] (full scan)
    int capacity, heads;
    int chunk;                 // positions per block (pooled scan); 0: the full scan sizes each
                               // sequence's runs from its live entries over gridDim.x blocks
    size_t key_stride;
    // full scan: per-block maximum keys [B][block_stride], or null
    uint32_t *block_keys;
    size_t block_stride;
    int block;                 // entries per pool block (divides 16)
    // pooled scan: pool [B][pool_blocks] ascending block indices (-1 unused);
    // output pairs [B][pool_blocks * block] (key 0 = no entry)
    const int32_t *pool;
    int pool_blocks;
    uint2 *out_pairs;
    // FP4 indexer keys: keys holds E2M1 codes (DI/2 bytes per row), scales
    // one E8M0 byte per 16 dims
    const uint8_t *idx_scales;
    int ratio;                 // tokens per entry of the cache
    float *out_scores = nullptr;   // full scan: [B][capacity] fp32 score of every live entry, or null
    uint32_t *tile_max = nullptr;  // full scan: [B][tile_stride] largest key of each 16-entry tile, or null
    size_t tile_stride = 0;
    // paged planes (page_size > 0): [n_pages][page_size] rows through the
    // block table [B][max_pages]
    const int32_t *block_table = nullptr;
    int page_size = 0, max_pages = 0, n_pages = 0;
};

// Paged scans resolve the pages of a block's run once, into kPageSlots
// words of the block's LDS array (the first row of each page); the grid
// keeps every run within kPageSlots - 2 pages.
constexpr int kPageSlots = 64;

// First plane row of page `lp` of sequence b (a table entry outside
// [0, n_pages) reads page 0: the scan only reads).
__device__ __forceinline__ int32_t page_row0(const ScanArgs &a, int b, int64_t lp)
{
    const int32_t pg = a.block_table[(size_t)b * a.max_pages + lp];
    return (pg >= 0 && pg < a.n_pages ? pg : 0) * a.page_size;
}

typedef __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; a field at its maximum does not wait).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (3 << 14) | (7 << 4);
constexpr int kNonTemporal = 2;     // cache policy of the streaming loads

constexpr int kPoolChunkMax = 4096;   // pool positions per block of the pooled scan

// Vector memory counter.  On this GPU stores count in vmcnt beside loads, so
// a ring wait that counts only the later tiles' loads would also wait for
// the stores issued after them, and with them for the next tile.  Every
// iteration of a scan loop therefore issues the same number of buffer stores
// from every lane (a masked lane gets an offset past its resource, an unused
// output a resource of no bytes).  With a ring of two, iteration i - 1
// issues tile i + 1's loads and its own stores after tile i's loads, in
// whichever order, so at the top of iteration i >= 1 tile i has landed once
// at most loads + stores are pending; tile 0 is waited for before the loop.
static_assert(kRing == 2, "the ring waits below count a ring of two tiles");
constexpr int scan_wait(int loads_per_tile, int stores) { return loads_per_tile + stores; }

__device__ __forceinline__ void store_b32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

// ReLU in one integer max: a float with its sign bit set (a negative value,
// -0) has a negative bit pattern and becomes +0, any other stays as it is.
// (fmaxf would first quiet a possible signalling NaN: two instructions.)
// A DMA of 16 or 4 bytes per lane from a buffer resource into LDS at dst
// (+ bytes * lane), non-temporal; an offset past the resource reads zeros.
// (Kept out of the kernels' bodies: the host compilation pass drops a kernel
// template whose body calls this builtin directly.)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voff, 0, 0, kNonTemporal);
}
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 4, voff, 0, 0, kNonTemporal);
}

__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Cross-lane reductions on the VALU (DPP and lane swaps, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Largest value of each 16-lane row, in every lane of the row (rotations).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t m)
{
    m = max(m, dpp_u32<0x128>(m));
    m = max(m, dpp_u32<0x124>(m));
    m = max(m, dpp_u32<0x122>(m));
    return max(m, dpp_u32<0x121>(m));
}

// Largest value of each aligned group of g lanes (g = 0, 1, 2, 4, 8 or 16),
// in every lane of the group: lane ^ 1 and lane ^ 2 by quad permutes, then
// the other quad of the eight and the other eight of the row by mirrors.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t m, int g)
{
    if (g >= 2) m = max(m, dpp_u32<0xB1>(m));
    if (g >= 4) m = max(m, dpp_u32<0x4E>(m));
    if (g >= 8) m = max(m, dpp_u32<0x141>(m));
    if (g >= 16) m = max(m, dpp_u32<0x140>(m));
    return m;
}

// (p_l + p_(l^16)) + (p_(l^32) + p_(l^48)): the sum over the four 16-lane
// rows at each column, in every lane (two lane swaps).
__device__ __forceinline__ float sum_rows(float p)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    const float s2 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s2), __float_as_uint(s2), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The outputs of a block's sequence as buffer resources (an unused output:
// no bytes).
struct ScanOut {
    __amdgpu_buffer_rsrc_t keys, scores, tmax, bkeys;
    int bsh;                    // log2 of the pool block (0 when none)
};

template <bool POOL>
__device__ __forceinline__ ScanOut scan_out(const ScanArgs &a, int b)
{
    ScanOut o;
    if constexpr (POOL) {
        const size_t n = (size_t)a.pool_blocks * a.block;
        o.keys = make_rsrc(a.out_pairs + (size_t)b * n, (uint32_t)(n * sizeof(uint2)));
        o.scores = o.tmax = o.bkeys = o.keys;
    } else {
        o.keys = make_rsrc(a.out_keys ? a.out_keys + (size_t)b * a.key_stride : nullptr,
                           a.out_keys ? (uint32_t)(a.key_stride * 4) : 0u);
        o.scores = make_rsrc(a.out_scores ? a.out_scores + (size_t)b * a.capacity : nullptr,
                             a.out_scores ? (uint32_t)a.capacity * 4u : 0u);
        o.tmax = make_rsrc(a.tile_max ? a.tile_max + (size_t)b * a.tile_stride : nullptr,
                           a.tile_max ? (uint32_t)(a.tile_stride * 4) : 0u);
        o.bkeys = make_rsrc(a.block_keys ? a.block_keys + (size_t)b * a.block_stride : nullptr,
                            a.block_keys ? (uint32_t)(a.block_stride * 4) : 0u);
    }
    o.bsh = a.block > 1 ? __builtin_ctz(a.block) : 0;
    return o;
}

// The epilogue of one lane for entry (pool position) e of the block's run,
// score p (live: e is a position of the run this lane reports; pe: the
// pooled scan's entry at e, read from LDS before the ring's refill): kStores
// buffer stores from every lane whatever is live (no branch around them).
template <bool POOL>
__device__ __forceinline__ void scan_store(const ScanArgs &a, const ScanOut &o, int32_t pe, int64_t e, bool live,
                                           bool tile_lane, float p)
{
    if constexpr (POOL) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = pe >= 0 ? u32x2_t{score_key(p), (uint32_t)pe} : u32x2_t{0u, 0xFFFFFFFFu};
        __builtin_amdgcn_raw_buffer_store_b64(v, o.keys, (int)(live ? (uint32_t)e * 8u : kMasked), 0, 0);
    } else {
        const uint32_t key = score_key(p);
        const uint32_t off = live ? (uint32_t)e * 4u : kMasked;
        store_b32(o.keys, off, key);
        store_b32(o.scores, off, __float_as_uint(p + 0.0f));
        // largest key of each 16-entry tile (entries past the end count as
        // key 0), written by the tile's first lane
        const uint32_t lk = live ? key : 0u;
        store_b32(o.tmax, tile_lane ? (uint32_t)(e >> 4) * 4u : kMasked, row_max_u32(lk));
        // largest key of each pool block (tiles start on block boundaries)
        const bool first = live && (e & ((1 << o.bsh) - 1)) == 0;
        store_b32(o.bkeys, first ? (uint32_t)(e >> o.bsh) * 4u : kMasked, group_max_u32(lk, a.block));
    }
}
template <bool POOL> constexpr int kStores = POOL ? 1 : 4;

// The query rows of the block's sequence (16 MT heads of DI bf16, zero rows
// past the heads) and the head weights (0 past the heads), staged once per
// block at the start of the LDS array, in the ring's space before any tile is
// issued; the waves take their MFMA operands from there.  (Loaded by every
// wave from L2 instead, 16 KB a wave, the start of a launch read some 32-50
// MB at once.)  Rows are DI bf16 plus 16 bytes, so the 16-byte reads of 16
// heads at one offset fall on distinct banks.
template <int DI> constexpr int kQRow = 2 * DI + 16;
template <int DI, int MT> constexpr int kQStage = 16 * MT * kQRow<DI> + 4 * 16 * MT;
template <int DI, int MT>
__device__ __forceinline__ void stage_query(const ScanArgs &a, int b, uint8_t *lds)
{
    constexpr int kPieces = DI / 8;                  // 16-byte pieces per row
    for (int i = threadIdx.x; i < 16 * MT * kPieces; i += kScanThreads) {
        const int h = i / kPieces, p = i % kPieces;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (h < a.heads) v = *reinterpret_cast<const u32x4_t *>(a.q + ((size_t)b * a.heads + h) * DI + 8 * p);
        *reinterpret_cast<u32x4_t *>(lds + h * kQRow<DI> + 16 * p) = v;
    }
    float *hws = reinterpret_cast<float *>(lds + 16 * MT * kQRow<DI>);
    if (threadIdx.x < 16 * MT) {
        const int h = threadIdx.x;
        hws[h] = h < a.heads ? (a.head_w ? a.head_w[(size_t)b * a.heads + h] : 1.0f) : 0.0f;
    }
}

// Run of block blockIdx.x over the n positions of its sequence: the pooled
// scan's fixed run length, or (full scan) the sequence's live entries cut
// into gridDim.x runs of a multiple of 64, so a cache allocated far beyond
// what it holds still spreads its entries over every block of the sequence.
__device__ __forceinline__ int64_t run_length(const ScanArgs &a, int64_t n)
{
    if (a.chunk > 0) return a.chunk;
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    return (per + 63) / 64 * 64;
}

// One block: a run of entries of one sequence (POOL: of pool positions);
// wave w takes 16-key tiles w, w + 4, ...  MT: 16-head row tiles of the
// query (1..4).
template <int DI, int MT, bool POOL, bool PAGED>
__global__ __launch_bounds__(kScanThreads, kScanBlocksPerCU) void indexer_scan_kernel(ScanArgs a)
{
    constexpr int kSteps = DI / 32;            // MFMA contraction steps per key
    constexpr int kRowBytes = 2 * DI;
    constexpr int kChunks = kRowBytes / 16;    // 16-byte chunks per key row
    constexpr int kTileBytes = 16 * kRowBytes;
    constexpr int kInst = kTileBytes / 1024;   // loads per tile (64 lanes x 16 B)
    // One LDS array: the wave rings, then (POOL) the entry of each position of
    // the run.  Reads of a different LDS object inside the loop would make the
    // compiler wait for every outstanding LDS DMA (vmcnt(0)) before them, which
    // serialises the ring; reads of the DMA's own object are left to the
    // explicit waits below.
    constexpr int kRingBytes = kScanWaves * kRing * kTileBytes;
    static_assert(kQStage<DI, MT> <= kRingBytes, "the query is staged in the ring's space");
    __shared__ __attribute__((aligned(16)))
    uint8_t lds[kRingBytes + (POOL ? 4 * kPoolChunkMax : 0) + (PAGED && !POOL ? 4 * kPageSlots : 0)];
    auto ring = reinterpret_cast<uint8_t (*)[kRing][kTileBytes]>(lds);
    int32_t *pool_rows = reinterpret_cast<int32_t *>(lds + kRingBytes);
    int32_t *pool_prow = pool_rows + kPoolChunkMax / 2;                     // PAGED and POOL
    int32_t *page_rows = reinterpret_cast<int32_t *>(lds + kRingBytes);     // PAGED, not POOL

    const int b = blockIdx.y;
    const int64_t E = entries_of(a.n_tokens, b, a.capacity, a.ratio);
    // the positions scanned: entries, or pool positions
    const int64_t N = POOL ? (E > 0 ? (int64_t)a.pool_blocks * a.block : 0) : E;
    const int64_t run = run_length(a, N);
    const int64_t e_begin = (int64_t)blockIdx.x * run;
    if (e_begin >= N) return;
    const int64_t e_end = N < e_begin + run ? N : e_begin + run;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int col = lane & 15, grp = lane >> 4;
    // PAGED: rows are plane rows; a tile's 16 entries lie in one page
    const int sh = PAGED ? __builtin_ctz(a.page_size) : 0;
    const int64_t first_page = e_begin >> sh;
    if constexpr (POOL) {
        // entry of every position of this block's run (-1: none) and, PAGED,
        // its plane row in the second half of the array (the run is at most
        // half as long); rows without an entry read row 0 and are dropped
        const int32_t *pl = a.pool + (size_t)b * a.pool_blocks;
        for (int i = threadIdx.x; i < e_end - e_begin; i += kScanThreads) {
            const int64_t p = e_begin + i;
            const int32_t blk = pl[p / a.block];
            const int64_t e = blk >= 0 ? (int64_t)blk * a.block + p % a.block : -1;
            pool_rows[i] = e < E ? (int32_t)e : -1;
            if constexpr (PAGED)
                pool_prow[i] = e >= 0 && e < E ? page_row0(a, b, e >> sh) + (int32_t)(e & (a.page_size - 1)) : 0;
        }
    } else if constexpr (PAGED) {
        const int n_pg = (int)(((e_end - 1) >> sh) - first_page + 1);
        for (int j = threadIdx.x; j < n_pg && j < kPageSlots; j += kScanThreads)
            page_rows[j] = page_row0(a, b, first_page + j);
    }
    stage_query<DI, MT>(a, b, lds);
    __syncthreads();

    const int n_tiles = (int)((e_end - e_begin + 15) / 16);
    const int my_n = n_tiles > w ? (n_tiles - w + kScanWaves - 1) / kScanWaves : 0;
    const uint8_t *kb = reinterpret_cast<const uint8_t *>(a.keys + (PAGED ? 0 : (size_t)b * a.capacity * DI));
    const ScanOut out = scan_out<POOL>(a, b);
    constexpr int kS = kStores<POOL>;
    constexpr int KI = kInst;                  // loads per tile

    // Tile i goes straight from HBM into LDS slot i % kRing with coalesced
    // 16-byte loads (instruction s covers bytes 1024 s .. 1024 s + 1023 of the
    // tile's 16 contiguous rows).  Lane l's bytes land at slot offset
    // 1024 s + 16 l; the lane fetches the chunk that belongs there under an
    // XOR swizzle (chunk c of row r at position c ^ (r % kChunks)), which
    // makes the operand reads below bank-conflict free.  Rows past the end
    // re-read the last valid row; their scores are dropped.
    auto issue = [&](int i) {
        const int64_t t0 = e_begin + (int64_t)(w + kScanWaves * i) * 16;
        uint8_t *slot = &ring[w][i % kRing][0];
        const bool tail = t0 + 16 > e_end;
#pragma unroll
        for (int s = 0; s < kInst; ++s) {
            const int u = 64 * s + lane, r = u / kChunks, p = u % kChunks, c = p ^ (r % kChunks);
            int64_t e = t0 + r;
            if (tail) e = e < e_end ? e : e_end - 1;
            if constexpr (POOL && PAGED) {
                e = pool_prow[e - e_begin];
            } else if constexpr (POOL) {
                const int32_t pe = pool_rows[e - e_begin];
                e = pe >= 0 ? pe : 0;
            } else if constexpr (PAGED) {
                const int64_t j = (e >> sh) - first_page;
                e = page_rows[j < kPageSlots ? j : kPageSlots - 1] + (e & (a.page_size - 1));
            }
            __builtin_amdgcn_global_load_lds((global_void_t *)(kb + (size_t)e * kRowBytes + 16 * c),
                                             (lds_void_t *)(slot + 1024 * s), 16, 0, kNonTemporal);
        }
    };

    // Indexer query as MFMA A operands: row = head, contraction slots
    // 8*grp..8*grp+7 of each 32-dim step; head weights of rows 4 grp ..
    // 4 grp + 3 of each head tile.  Missing heads: zero rows, weight 0.
    u32x4_t qa[MT][kSteps];
    float hw[MT][4];
    const float *hws = reinterpret_cast<const float *>(lds + 16 * MT * kQRow<DI>);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint8_t *qrow = lds + (16 * mt + col) * kQRow<DI>;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) qa[mt][s] = *reinterpret_cast<const u32x4_t *>(qrow + 16 * (4 * s + grp));
        const float4 h4 = *reinterpret_cast<const float4 *>(hws + 16 * mt + 4 * grp);
        hw[mt][0] = h4.x; hw[mt][1] = h4.y; hw[mt][2] = h4.z; hw[mt][3] = h4.w;
    }
    __syncthreads();                                // the ring may now overwrite the staged query
#pragma unroll
    for (int i = 0; i < kRing; ++i) issue(i);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(KI * (kRing - 1)));             // tile 0 has landed

    for (int i = 0; i < my_n; ++i) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(scan_wait(KI, kS)));       // tile i has landed
        const uint8_t *slot = &ring[w][i % kRing][0];
        u32x4_t bop[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int p = (4 * s + grp) ^ (col % kChunks);
            bop[s] = *reinterpret_cast<const u32x4_t *>(slot + 16 * (col * kChunks + p));
        }
        // lanes 0-15 report the tile's 16 entries
        const int64_t e = e_begin + (int64_t)(w + kScanWaves * i) * 16 + lane;
        const bool live = lane < 16 && e < e_end;
        const int32_t pe = POOL ? pool_rows[live ? e - e_begin : 0] : 0;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);      // slot read before it is refilled
        issue(i + kRing);
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32(qa[mt][s], bop[s], acc[mt]);
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) part += hw[mt][v] * relu(acc[mt][v]);
        part = sum_rows(part);
        scan_store<POOL>(a, out, pe, e, live, lane == 0, part);
    }
    // no LDS write may land after the block's LDS is handed to another block
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// The scan over FP4 indexer keys (E2M1 codes + one E8M0 scale per 16 dims,
// the pages' 72-byte key at DI = 128).  Tiles of 64 keys: a tile's codes
// (DI/2 bytes per key, XOR-swizzled 16-byte chunks as in the bf16 scan) and
// scales (DI/16 bytes per key) go by DMA into the wave's LDS slot.  The
// contraction order is permuted: at step s, lane group g holds dims
// 8 (kSteps g + s) .. + 7, so a lane's code words for all steps are one
// contiguous piece of the key row (one LDS read) and its scale bytes are
// adjacent; the query is loaded in the same order.  Each 16-key column tile
// is converted to bf16 by the hardware FP4 conversion, which applies the
// group's power-of-two scale exactly, and goes through the same bf16 MFMA
// and epilogue as the bf16 scan.
template <int DI, int MT, bool POOL, bool PAGED, bool DENSE = false>
__global__ __launch_bounds__(kScanThreads, kScanBlocksPerCU) void indexer_scan_fp4_kernel(ScanArgs a)
{
    static_assert(!DENSE || (!POOL && !PAGED), "dense rows are neither pooled nor paged");
    constexpr int kSteps = DI / 32;
    constexpr int kTileKeys = 64;
    constexpr int kCodeBytes = DI / 2;                   // per key
    constexpr int kScaleBytes = DI / 16;                 // per key
    constexpr int kChunks = kCodeBytes / 16;             // 16-byte chunks per key row
    constexpr int kTileCode = kTileKeys * kCodeBytes;
    constexpr int kTileScale = kTileKeys * kScaleBytes;
    constexpr int kInstC = kTileCode / 1024;             // 16-byte DMA per lane
    constexpr int kInstS = kTileScale / 256;             // 4-byte DMA per lane
    constexpr int kPiece = 4 * kSteps;                   // bytes of a lane's code piece
    static_assert(kInstC >= 1 && kInstS >= 1, "tile sizes");
    // One LDS array (see the bf16 scan): the wave rings, then (POOL) the
    // entry of each position of the run.
    constexpr int kRingBytes = kScanWaves * kRing * (kTileCode + kTileScale);
    static_assert(kQStage<DI, MT> <= kRingBytes, "the query is staged in the ring's space");
    __shared__ __attribute__((aligned(16)))
    uint8_t lds[kRingBytes + (POOL ? 4 * kPoolChunkMax : 0) + (PAGED && !POOL ? 4 * kPageSlots : 0)];
    auto ring = reinterpret_cast<uint8_t (*)[kRing][kTileCode + kTileScale]>(lds);
    int32_t *pool_rows = reinterpret_cast<int32_t *>(lds + kRingBytes);
    int32_t *pool_prow = pool_rows + kPoolChunkMax / 2;                     // PAGED and POOL
    int32_t *page_rows = reinterpret_cast<int32_t *>(lds + kRingBytes);     // PAGED, not POOL

    const int b = blockIdx.y;
    const int64_t E = entries_of(a.n_tokens, b, a.capacity, a.ratio);
    const int64_t N = POOL ? (E > 0 ? (int64_t)a.pool_blocks * a.block : 0) : E;
    const int64_t run = run_length(a, N);
    const int64_t e_begin = (int64_t)blockIdx.x * run;
    if (e_begin >= N) return;
    const int64_t e_end = N < e_begin + run ? N : e_begin + run;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int col = lane & 15, grp = lane >> 4;
    // PAGED: rows are plane rows; a tile's 64 entries lie in one page
    const int sh = PAGED ? __builtin_ctz(a.page_size) : 0;
    const int64_t first_page = e_begin >> sh;
    if constexpr (POOL) {
        const int32_t *pl = a.pool + (size_t)b * a.pool_blocks;
        for (int i = threadIdx.x; i < e_end - e_begin; i += kScanThreads) {
            const int64_t p = e_begin + i;
            const int32_t blk = pl[p / a.block];
            const int64_t e = blk >= 0 ? (int64_t)blk * a.block + p % a.block : -1;
            pool_rows[i] = e < E ? (int32_t)e : -1;
            if constexpr (PAGED)
                pool_prow[i] = e >= 0 && e < E ? page_row0(a, b, e >> sh) + (int32_t)(e & (a.page_size - 1)) : 0;
        }
    } else if constexpr (PAGED) {
        const int n_pg = (int)(((e_end - 1) >> sh) - first_page + 1);
        for (int j = threadIdx.x; j < n_pg && j < kPageSlots; j += kScanThreads)
            page_rows[j] = page_row0(a, b, first_page + j);
    }
    stage_query<DI, MT>(a, b, lds);
    __syncthreads();

    const int n_tiles = (int)((e_end - e_begin + kTileKeys - 1) / kTileKeys);
    const int my_n = n_tiles > w ? (n_tiles - w + kScanWaves - 1) / kScanWaves : 0;
    const uint8_t *kb = reinterpret_cast<const uint8_t *>(a.keys) + (PAGED ? 0 : (size_t)b * a.capacity * kCodeBytes);
    const uint8_t *sb = a.idx_scales + (PAGED ? 0 : (size_t)b * a.capacity * kScaleBytes);

    // cache row of position e (clamped into the run; positions without an
    // entry read row 0 and are dropped)
    auto row_of = [&](int64_t e) -> int64_t {
        e = e < e_end ? e : e_end - 1;
        if constexpr (POOL && PAGED) {
            return pool_prow[e - e_begin];
        } else if constexpr (POOL) {
            const int32_t pe = pool_rows[e - e_begin];
            return pe >= 0 ? pe : 0;
        } else if constexpr (PAGED) {
            const int64_t j = (e >> sh) - first_page;
            return page_rows[j < kPageSlots ? j : kPageSlots - 1] + (e & (a.page_size - 1));
        } else {
            return e;
        }
    };
    // DENSE (the host's choice for rows neither pooled nor paged whose run
    // offsets fit 31 bits): codes and scales through two buffer resources
    // over the block's run; a lane's offsets within a tile are fixed (load s
    // adds 1024 s, or 256 s for the scales), one 32-bit add places the tile,
    // and rows past the run lie outside the resources and read as zeros (their
    // scores are dropped).  Otherwise each row comes from row_of.
    const __amdgpu_buffer_rsrc_t crs =
        make_rsrc(kb + (size_t)e_begin * kCodeBytes, DENSE ? (uint32_t)((e_end - e_begin) * kCodeBytes) : 0u);
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(sb + (size_t)e_begin * kScaleBytes, DENSE ? (uint32_t)((e_end - e_begin) * kScaleBytes) : 0u);
    const uint32_t coff = (uint32_t)((w * kTileKeys + lane / kChunks) * kCodeBytes +
                                     16 * ((lane % kChunks) ^ ((lane / kChunks) % kChunks)));
    const uint32_t soff = (uint32_t)((w * kTileKeys + 4 * lane / kScaleBytes) * kScaleBytes + (4 * lane) % kScaleBytes);
    auto issue = [&](int i) {
        uint8_t *slot = &ring[w][i % kRing][0];
        if constexpr (DENSE) {
            const uint32_t tk = (uint32_t)(kScanWaves * i) * kTileKeys;
#pragma unroll
            for (int s = 0; s < kInstC; ++s) load_lds16(crs, slot + 1024 * s, coff + tk * kCodeBytes + 1024 * s);
#pragma unroll
            for (int s = 0; s < kInstS; ++s)
                load_lds4(srs, slot + kTileCode + 256 * s, soff + tk * kScaleBytes + 256 * s);
            return;
        }
        const int64_t t0 = e_begin + (int64_t)(w + kScanWaves * i) * kTileKeys;
#pragma unroll
        for (int s = 0; s < kInstC; ++s) {
            const int u = 64 * s + lane, r = u / kChunks, p = u % kChunks, c = p ^ (r % kChunks);
            __builtin_amdgcn_global_load_lds((global_void_t *)(kb + (size_t)row_of(t0 + r) * kCodeBytes + 16 * c),
                                             (lds_void_t *)(slot + 1024 * s), 16, 0, kNonTemporal);
        }
#pragma unroll
        for (int s = 0; s < kInstS; ++s) {
            const int u = 4 * (64 * s + lane), r = u / kScaleBytes, o = u % kScaleBytes;
            __builtin_amdgcn_global_load_lds((global_void_t *)(sb + (size_t)row_of(t0 + r) * kScaleBytes + o),
                                             (lds_void_t *)(slot + kTileCode + 256 * s), 4, 0, kNonTemporal);
        }
    };

    const ScanOut out = scan_out<POOL>(a, b);
    constexpr int kS = kStores<POOL>;
    constexpr int KI = kInstC + kInstS;        // loads per tile
    // head weights of rows 4 grp .. 4 grp + 3 of each head tile, in registers
    // (an LDS read after the ring's refill would wait for the refill), and the
    // query in the permuted contraction order, both from the staged copy
    const float *hws = reinterpret_cast<const float *>(lds + 16 * MT * kQRow<DI>);
    float4 hw4[MT];
    u32x4_t qa[MT][kSteps];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        hw4[mt] = *reinterpret_cast<const float4 *>(hws + 16 * mt + 4 * grp);
        const uint8_t *qrow = lds + (16 * mt + col) * kQRow<DI>;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            qa[mt][s] = *reinterpret_cast<const u32x4_t *>(qrow + 16 * (kSteps * grp + s));
    }
    __syncthreads();                                // the ring may now overwrite the staged query
#pragma unroll
    for (int i = 0; i < kRing; ++i) issue(i);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(KI * (kRing - 1)));             // tile 0 has landed

    for (int i = 0; i < my_n; ++i) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(scan_wait(KI, kS)));       // tile i has landed
        const uint8_t *slot = &ring[w][i % kRing][0];
        uint32_t cw[4][kSteps];
        uint32_t sw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = 16 * j + col;
            const int byte0 = kPiece * grp, p = (byte0 >> 4) ^ (key % kChunks);
            const uint8_t *src = slot + key * kCodeBytes + 16 * p + (byte0 & 15);
            if constexpr (kSteps == 4) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src);
                cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                cw[j][0] = v.x; cw[j][1] = v.y;
            }
            const uint8_t *ss = slot + kTileCode + key * kScaleBytes;
            sw[j] = kSteps == 4 ? (uint32_t)*reinterpret_cast<const uint16_t *>(ss + 2 * grp) : (uint32_t)ss[grp];
        }
        const int64_t t0 = e_begin + (int64_t)(w + kScanWaves * i) * kTileKeys;
        // lane l reports entry t0 + l: column l % 16 of column tile l / 16
        const int64_t e = t0 + lane;
        const bool live = e < e_end;
        const int32_t pe = POOL ? pool_rows[live ? e - e_begin : 0] : 0;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);      // slot read before it is refilled
        issue(i + kRing);
        float pj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4_t acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const uint32_t byte = kSteps == 4 ? (sw[j] >> (8 * (s >> 1))) & 0xFFu : sw[j];
                const u32x4_t bop = fp4x8_scaled_to_bf16x8(cw[j][s], e8m0_to_f32(byte));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32(qa[mt][s], bop, acc[mt]);
            }
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 hw = hw4[mt];
                part += hw.x * relu(acc[mt][0]);
                part += hw.y * relu(acc[mt][1]);
                part += hw.z * relu(acc[mt][2]);
                part += hw.w * relu(acc[mt][3]);
            }
            pj[j] = sum_rows(part);
        }
        const float pm = grp == 0 ? pj[0] : grp == 1 ? pj[1] : grp == 2 ? pj[2] : pj[3];
        scan_store<POOL>(a, out, pe, e, live, col == 0, pm);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

}  // namespace

// Blocks per sequence and positions per block for n positions per sequence:
// one round of blocks, runs a multiple of 64 (and at most `cap`), 3 blocks
// per CU (what registers and LDS allow).  With the query staged once per
// block and 3 blocks per CU, the 64K x 32 step runs 1.3% faster than with
// every wave loading the query and 2 blocks per CU (10,372 against 10,242
// steps/s on one box), the 128K x 64 group 0.7% slower (1,616 against
// 1,629: longer runs amortise the loads); with every wave loading it, 3
// blocks per CU had been slower at 64K x 32 (the launch's start reading
// 50 MB of queries from L2); a ragged
// 256-sequence batch was faster with 3 either way (116 us against 156 with
// 2, where fewer runs per sequence leave the long sequences' blocks with
// most of the work), and so are FP4 keys, whose scan is bound by its per-key
// arithmetic.
static int scan_blocks_per_cu(const cskv_cache &) { return kScanBlocksPerCU; }
static int scan_blocks_per_seq(int batch, int per_cu)
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    const int slots = per_cu * cus;
    return batch >= slots ? 1 : slots / batch;
}
static int scan_chunk(int batch, size_t n, size_t cap, int per_cu)
{
    const int per_seq = scan_blocks_per_seq(batch, per_cu);
    size_t chunk = (n + per_seq - 1) / per_seq;
    chunk = (chunk + 63) / 64 * 64;
    return (int)(chunk < cap ? chunk : cap);
}

template <bool POOL, bool PAGED>
static void scan_dispatch_t(const cskv_cache &c, int heads, const ScanArgs &sa, dim3 grid, hipStream_t s)
{
    const int mt = (heads + 15) / 16;
    const TimedLaunch ts = timer_take(CSKV_KERNEL_INDEXER_SCAN);
    auto scan = [&](auto kernel) { launch_kernel(kernel, grid, dim3(kScanThreads), s, ts.start, ts.stop, sa); };
    if (c.idx_format == CSKV_IDX_FP4) {
        // dense rows whose byte offsets within a sequence fit 31 bits
        constexpr bool kCanDense = !POOL && !PAGED;
        if (kCanDense && (uint64_t)c.capacity * (uint64_t)(c.idx_dim / 2) < (1ull << 31)) {
            constexpr bool D = kCanDense;
            if (c.idx_dim == 128) {
                if (mt == 4) scan(indexer_scan_fp4_kernel<128, 4, POOL, PAGED, D>);
                else if (mt == 3) scan(indexer_scan_fp4_kernel<128, 3, POOL, PAGED, D>);
                else if (mt == 2) scan(indexer_scan_fp4_kernel<128, 2, POOL, PAGED, D>);
                else scan(indexer_scan_fp4_kernel<128, 1, POOL, PAGED, D>);
            } else {
                if (mt == 4) scan(indexer_scan_fp4_kernel<64, 4, POOL, PAGED, D>);
                else if (mt == 3) scan(indexer_scan_fp4_kernel<64, 3, POOL, PAGED, D>);
                else if (mt == 2) scan(indexer_scan_fp4_kernel<64, 2, POOL, PAGED, D>);
                else scan(indexer_scan_fp4_kernel<64, 1, POOL, PAGED, D>);
            }
            return;
        }
        if (c.idx_dim == 128) {
            if (mt == 4) scan(indexer_scan_fp4_kernel<128, 4, POOL, PAGED>);
            else if (mt == 3) scan(indexer_scan_fp4_kernel<128, 3, POOL, PAGED>);
            else if (mt == 2) scan(indexer_scan_fp4_kernel<128, 2, POOL, PAGED>);
            else scan(indexer_scan_fp4_kernel<128, 1, POOL, PAGED>);
        } else {
            if (mt == 4) scan(indexer_scan_fp4_kernel<64, 4, POOL, PAGED>);
            else if (mt == 3) scan(indexer_scan_fp4_kernel<64, 3, POOL, PAGED>);
            else if (mt == 2) scan(indexer_scan_fp4_kernel<64, 2, POOL, PAGED>);
            else scan(indexer_scan_fp4_kernel<64, 1, POOL, PAGED>);
        }
        return;
    }
    if (c.idx_dim == 128) {
        if (mt == 4) scan(indexer_scan_kernel<128, 4, POOL, PAGED>);
        else if (mt == 3) scan(indexer_scan_kernel<128, 3, POOL, PAGED>);
        else if (mt == 2) scan(indexer_scan_kernel<128, 2, POOL, PAGED>);
        else scan(indexer_scan_kernel<128, 1, POOL, PAGED>);
    } else {
        if (mt == 4) scan(indexer_scan_kernel<64, 4, POOL, PAGED>);
        else if (mt == 3) scan(indexer_scan_kernel<64, 3, POOL, PAGED>);
        else if (mt == 2) scan(indexer_scan_kernel<64, 2, POOL, PAGED>);
        else scan(indexer_scan_kernel<64, 1, POOL, PAGED>);
    }
}

template <bool POOL>
static void scan_dispatch(const cskv_cache &c, int heads, const ScanArgs &sa, dim3 grid, hipStream_t s)
{
    if (c.page_size > 0) scan_dispatch_t<POOL, true>(c, heads, sa, grid, s);
    else scan_dispatch_t<POOL, false>(c, heads, sa, grid, s);
}

void launch_indexer_scan(const cskv_cache &c, const uint16_t *q_idx, int heads, const float *head_w,
                         uint32_t *keys, hipStream_t s, uint32_t *block_keys, size_t block_stride, int block,
                         float *out_scores, uint32_t *tile_max, size_t tile_stride)
{
    // per sequence one round's share of the chip's blocks, each run sized on
    // the device from the sequence's live entries (never more blocks than
    // 64-entry runs fit in the capacity)
    const int per_seq = scan_blocks_per_seq(c.batch, scan_blocks_per_cu(c));
    const size_t max_runs = ((size_t)c.capacity + 63) / 64;
    size_t gxs = (size_t)per_seq < max_runs ? (size_t)per_seq : max_runs;
    if (c.page_size > 0) {
        // paged: every run within kPageSlots - 2 pages (a run may start inside a page)
        const size_t span = (size_t)(kPageSlots - 3) * c.page_size;
        const size_t need = ((size_t)c.capacity + span - 1) / span;
        gxs = gxs > need ? gxs : need;
    }
    const unsigned gx = (unsigned)gxs;
    ScanArgs sa{c.idx_keys, c.n_tokens, q_idx, head_w, keys, c.capacity, heads, 0, score_key_stride(c),
                block_keys, block_stride, block, nullptr, 0, nullptr, c.idx_scales, c.ratio, out_scores,
                tile_max, tile_stride, c.block_table, c.page_size, c.max_pages, c.n_pages};
    dim3 grid(gx, (unsigned)c.batch);
    scan_dispatch<false>(c, heads, sa, grid, s);
}

void launch_pool_scan(const cskv_cache &c, const uint16_t *q_idx, int heads, const float *head_w,
                      const int32_t *pool, int pool_blocks, int block, uint2 *pairs, hipStream_t s)
{
    const size_t n = (size_t)pool_blocks * block;
    // paged: half the positions per block, the other half of the block's
    // position array holds their plane rows
    const int chunk = scan_chunk(c.batch, n, c.page_size > 0 ? kPoolChunkMax / 2 : kPoolChunkMax,
                                 scan_blocks_per_cu(c));
    ScanArgs sa{c.idx_keys, c.n_tokens, q_idx, head_w, nullptr, c.capacity, heads, chunk, 0,
                nullptr, 0, block, pool, pool_blocks, pairs, c.idx_scales, c.ratio, nullptr,
                nullptr, 0, c.block_table, c.page_size, c.max_pages, c.n_pages};
    dim3 grid((unsigned)((n + chunk - 1) / chunk), (unsigned)c.batch);
    scan_dispatch<true>(c, heads, sa, grid, s);
}

}  // namespace cskv
